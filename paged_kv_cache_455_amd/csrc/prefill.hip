// Mixed continuous-batching step: chunked prefills and decodes in one launch.
//
// uml.org.cn "Continuous Batching": new requests' prefill work and running
// requests' decode steps share one batch.  5688vip chapter 3, section 3.1:
// generation is autoregressive, so query row i of a chunk that extends a
// sequence to seq_len tokens sits at position seq_len - q_len + i and attends to
// keys 0 .. that position.
//
// For f16 / bf16 KV the step is two launches (after a small one that lists the
// prefill tiles on the device, heaviest first over the whole step):
//  * prefill tiles: 64 * RB query rows -- (token, head) pairs of one kv head's GQA
//    group -- against 32-key steps of the chunk's context, with the dense products
//    on MFMA (v_mfma_f32_16x16x32_{f16,bf16}):
//      S^T = K . Q^T   (A = 16 keys x 32 dims from LDS, B = q rows in registers)
//      O^T += V^T . P^T (A = 16 dims x 32 keys of V: V sits in LDS row-major like
//                        K, and gfx950's transposed 16-bit LDS read hands each lane
//                        the key-consecutive values of one dim; B = the
//                        probabilities straight from S^T's registers)
//    The two QK products of a step take their 16 key rows in an interleaved order
//    (first: keys 8(r/4) + r%4, second: the same + 4) so that each lane's 8 scores
//    are the 8 consecutive keys its P^T operand needs; computing O^T rather than O
//    keeps each query row's running max, sum and rescale inside one lane; the
//    running sums come from the matrix cores too, as ones . P^T.  For bf16 KV, P
//    enters both products as two 16-bit parts, hi + lo (p_operands), so the weights
//    are not rounded to bf16's 8 bits.
//  * decode rows (q_len == 1): the balanced-split decode of decode_impl.h over
//    the batch's one-token sequences (query row qsl[s]), with its piece merge.
// Other KV types run every query row through the partitioned decode path.
#include <type_traits>

#include "decode_impl.h"

namespace pa {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kRowBlocks = 2;                   // 16-row MFMA blocks per wave
constexpr int kTileRows = 4 * 16 * kRowBlocks;  // query rows (token, head) per prefill workgroup
constexpr int kKeyStep = 32;    // keys per step (two blocks)
constexpr int kItemBits = 12;   // item = (sequence << 12) | tile or partition index
// key steps whose K/V loads are in flight in registers (3 would need more than 256
// VGPRs at head_dim 128: one workgroup per CU instead of two)
constexpr int kStages = 2;
constexpr float kLazy = 8.f;    // running-max slack before a rescale (log2 units)

int mixed_tile_rows() { return kTileRows; }

template <int D>
struct PrefillLds {
  static constexpr int kKHalves = kKeyStep * D;     // K: [32 keys][D], chunks swizzled
  static constexpr int kVHalves = kKeyStep * D;     // V: [32 keys][D], chunks swizzled
  static constexpr int kBufHalves = kKHalves + kVHalves;
  static constexpr int kBytes = 2 * kBufHalves * 2;  // two K/V buffers
};

template <int KV>
__device__ __forceinline__ f4_t mfma32(const u32x4 &a, const u32x4 &b, const f4_t &c) {
  if constexpr (KV == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
}

typedef float f2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h2v_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2v_t __attribute__((ext_vector_type(2)));

// P^T operands of 8 probabilities.  The P.V product and the row sums see the same
// operands, so the output is sum(p~ v) / sum(p~) for the weights p~ as the MFMA
// inputs hold them.
//  f16: p rounded to nearest even (lo unused).  Each weight then carries a
//       relative error below 2^-11, which moves the output by less than 2^-11 of
//       the weighted spread |v - out| of the values -- the order of V's own f16
//       storage precision, and inside the f16 tolerance (a simulation of 25.6 M
//       outputs on unscaled N(0,1) data, few to hundreds of keys, peaked at 0.72
//       of the bar: max(2e-3, one ulp)).
//  bf16: one rounding would be 2^-8 relative (3x the bar on such data), so p is
//       split into two parts, p ~= hi + lo: hi = p truncated to its upper 16 bits
//       (a byte permute of two values), lo = (p - hi) rounded to nearest even, the
//       difference exact in fp32; the pair holds p to 2^-15 relative and every
//       product runs twice (hi, then lo).
template <int KV>
constexpr bool kSplitP = KV == PA_BF16;

template <int KV>
__device__ __forceinline__ void p_operands(const float *p, u32x4 &hi, u32x4 &lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = p[2 * i], b = p[2 * i + 1];
    if constexpr (!kSplitP<KV>) {
      hi[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2v_t));
    } else {
      const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
      hi[i] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // upper halves of a (low), b (high)
      const float ra = a - __builtin_bit_cast(float, ua & 0xFFFF0000u);
      const float rb = b - __builtin_bit_cast(float, ub & 0xFFFF0000u);
      lo[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{ra, rb}, b2v_t));
    }
  }
}

// gfx950's transposed LDS read of 16-bit values (ds_read_b64_tr_b16).  Each lane
// names 8 bytes; inside each 16-lane group, lane i receives element i % 4 of the
// reads of lanes 4e + i / 4 (e = 0 .. 3).  So when those lanes read 4 rows of a
// row-major tile, 4 lanes per row side by side over 16 columns, lane i gets
// column i of the 4 rows.
typedef short s4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const _Float16 *p) {
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4_t *)p));
}

// XOR swizzle of a K row's 16-byte chunks (a value below D/8).  A K operand read
// takes, in each 16-lane group, the same chunk of keys 8(c/4) + c%4 (c = 0..15;
// +4 for the second product); the swizzle gives those 16 rows distinct bank ranges
// per 16 lanes, and per 8, with 64 or 32 four-byte banks (key % (D/8), its simpler
// form, left keys k and k + 16 on one range).  Row writes stay a permutation.
template <int D>
__device__ __forceinline__ int k_swizzle(int key) {
  static_assert(D == 64 || D == 128, "prefill tiles take head_dim 64 or 128");
  if constexpr (D == 128)
    return (key & 3) | (((key >> 3) & 3) << 2);
  else
    return ((key >> 1) & 1) | (((key >> 3) & 1) << 1) | (((key & 1) ^ ((key >> 4) & 1)) << 2);
}

// XOR swizzle of a V row's 16-byte chunks (an even value below D/8).  A
// transposed V operand read touches keys 8g + r (g = 0..3, r = 0..3; +4 for its
// second half) at the same two chunks of every row; the swizzle puts each half
// wave's 8 rows on 8 disjoint 32-byte bank ranges (and each 16-lane group's 4 rows
// on 4), with 32 or 64 four-byte banks.  Row writes stay a permutation of chunks.
template <int D>
__device__ __forceinline__ int v_swizzle(int key) {
  static_assert(D == 64 || D == 128, "prefill tiles take head_dim 64 or 128");
  if constexpr (D == 128)
    return 2 * ((key & 3) | (((key >> 3) & 1) << 2));
  else
    return 2 * ((((key >> 1) & 1) | (((key >> 3) & 1) << 1)) ^ ((key & 1) << 1));
}

// One prefill tile: query tokens [qt*QTOK, ...) of sequence s, kv head h.
// Rows: wave w, row block rb, lane column c16 -> row (w*RB + rb)*16 + c16 = token*G + head.
// Pipeline, per 32-key step n (NS = kStages): the two block-table entries of step
// n+NS+1 are read, K/V of step n+NS are loaded into registers, step n is computed
// from LDS and step n+1 is written to the other LDS buffer.  Every load is issued unconditionally
// (indices clamped to the tile's last block, keys past its reach zeroed when they
// reach LDS) so that the compiler's waits count loads instead of draining them.
// Each K or V operand read from LDS serves all RB row blocks of the wave.
template <int KV, int D, int G>
__device__ __forceinline__ void prefill_tile(const MixedArgs &a, int s, int h, int qt,
                                             char *smem) {
  constexpr int RB = kRowBlocks;
  constexpr int QTOK = kTileRows / G;
  constexpr int NKK = D / 32;        // QK MFMAs along head_dim
  constexpr int NSL = D / 16;        // 16-dim output slices
  constexpr int CPR = D / 8;         // 16-byte chunks per key row
  constexpr int NCH = kKeyStep * CPR / 256;  // K (and V) chunks per thread per step
  using L = PrefillLds<D>;
  _Float16 *lds = reinterpret_cast<_Float16 *>(smem);
  const DecodeArgs &d = a.dec;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the wave's bounds stay scalar
  const int g16 = lane >> 4, c16 = lane & 15;
  const int q0 = a.qsl[s], q_len = a.qsl[s + 1] - q0;
  const int first_pos = d.ctx[s] - q_len;
  const int t0 = qt * QTOK;
  const int t_end = min(t0 + QTOK, q_len);
  const int nkeys = first_pos + t_end;  // keys any row of the tile can see
  const int32_t *bt = d.bt + (int64_t)s * d.max_blocks_per_seq;
  const int Hq = d.num_q_heads, Hkv = d.num_kv_heads;
  // the wave's rows: tokens t0 + (wave*RB*16) / G ... ; positions bound its keys
  const int wave_tok0 = t0 + (wave * RB * 16) / G;
  const int wave_min_pos = first_pos + wave_tok0;
  const int wave_max_pos = first_pos + min(t0 + ((wave + 1) * RB * 16 - 1) / G, q_len - 1);

  const int nblk = (nkeys + kBlock - 1) / kBlock;

  // query operands: lane (row c16 of row block rb) holds dims 32*kk + 8*g16 .. +8
  u32x4 qop[RB][NKK];
  int row_pos[RB];
  bool row_ok[RB];
  int64_t row_out[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = (wave * RB + rb) * 16 + c16;
    const int tok = t0 + row / G, g = row % G;
    row_ok[rb] = tok < q_len;
    row_pos[rb] = row_ok[rb] ? first_pos + tok : -1;
    row_out[rb] = ((int64_t)(q0 + tok) * Hq + h * G + g) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qop[rb][kk] = u32x4{0, 0, 0, 0};
    if (row_ok[rb]) {  // rows past the chunk's end are never read
      const char *qp = reinterpret_cast<const char *>(d.q) + row_out[rb] * 2;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        qop[rb][kk] = *reinterpret_cast<const u32x4 *>(qp + (32 * kk + 8 * g16) * 2);
    }
  }

  // o: O^T slices; lsum: the running softmax denominators, accumulated on the matrix
  // cores as ones(16 x 32) . P^T (hi and lo parts for bf16), so every element holds
  // its query row's sum of the probabilities as the P.V product used them
  f4_t o[RB][NSL], lsum[RB];
  float m[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    lsum[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) o[rb][sl] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr uint32_t kOne2 = KV == PA_F16 ? 0x3C003C00u : 0x3F803F80u;  // two 16-bit 1.0s
  const u32x4 ones = u32x4{kOne2, kOne2, kOne2, kOne2};

  // ---- global -> registers -> LDS staging of one 32-key step ----
  const char *kpool = reinterpret_cast<const char *>(d.k);
  const char *vpool = reinterpret_cast<const char *>(d.v);
  // 16-row tile indices of step n's two tiles (clamped to the last tile)
  struct StepBt {
    int64_t u0, u1;
  };
  const int sh = d.bs_shift;
  auto bt_load = [&](int n) {
    const int j0 = min(2 * n, nblk - 1), j1 = min(2 * n + 1, nblk - 1);
    StepBt r;
    r.u0 = tile_index(bt[j0 >> sh], Hkv, h, j0, sh);
    r.u1 = tile_index(bt[j1 >> sh], Hkv, h, j1, sh);
    return r;
  };
  // K and V alike: chunk q of the step = key q / CPR, 16-byte column q % CPR
  // (a wave's loads of one key row are contiguous).
  struct Stage {
    u32x4 k[NCH], v[NCH];
  };
  // Which of the step's two 16-row tiles a thread's chunk sits in is the same for
  // the whole wave (2*D key-row chunks per tile is a multiple of 64 lanes), so it is
  // chosen on the scalar unit from the wave's first thread; the thread's offset
  // inside the tile is fixed.
  const int wtid = __builtin_amdgcn_readfirstlane(tid);
  uint32_t k_off[NCH];
  bool k_hi[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int q = tid + 256 * c;
    k_off[c] = (uint32_t)(((q / CPR) % kBlock) * D * 2 + (q % CPR) * 16);
    k_hi[c] = (wtid + 256 * c) / CPR >= kBlock;
  }
  auto gload = [&](const StepBt &b, Stage &st) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int64_t tile = (k_hi[c] ? b.u1 : b.u0) * (int64_t)(kBlock * D * 2);
      st.k[c] = *reinterpret_cast<const u32x4 *>(kpool + tile + k_off[c]);
      st.v[c] = *reinterpret_cast<const u32x4 *>(vpool + tile + k_off[c]);
    }
  };
  // Both go to LDS as 16-byte chunks, row-major, swizzled so that the operand reads
  // spread over the banks (K by k_swizzle, V by v_swizzle).  Keys at or past nkeys
  // (the tile's reach; they may hold anything, NaN included) are zeroed on the way in.
  auto lstore_impl = [&](int buf, int kb, const Stage &st, auto masked) {
    _Float16 *K = lds + buf * L::kBufHalves;
    _Float16 *V = K + L::kKHalves;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + 256 * c;
      const int key = q / CPR, cc = q % CPR;
      const bool ok = !masked.value || kb + key < nkeys;
      const u32x4 zero = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4 *>(K + key * D + (cc ^ k_swizzle<D>(key)) * 8) = ok ? st.k[c] : zero;
      *reinterpret_cast<u32x4 *>(V + key * D + (cc ^ v_swizzle<D>(key)) * 8) = ok ? st.v[c] : zero;
    }
  };
  // only a step that reaches past the tile's keys needs the zeroing (a uniform branch)
  auto lstore = [&](int buf, int kb, const Stage &st) {
    if (kb + kKeyStep <= nkeys)
      lstore_impl(buf, kb, st, std::false_type{});
    else
      lstore_impl(buf, kb, st, std::true_type{});
  };

  const int key1 = 8 * (c16 >> 2) + (c16 & 3);  // key row of this lane in QK product 1
  const int key2 = key1 + 4;                      // ... in product 2
  // V^T operand of slice sl: this lane reads dims 16 sl + vcol .. +3 of key rows
  // vrow (keys 8 g16 .. +3 of the operand) and vrow + 4 (keys + 4 .. +7); the
  // transposed read returns dim 16 sl + c16 of the 4 keys.  vrow + 4 shares vrow's
  // swizzle (bit 2 of the key is not in it).
  const int vrow = 8 * g16 + (c16 >> 2), vcol = 4 * (c16 & 3);
  // One 32-key step from LDS buffer buf (keys kb ..): S^T = K . Q^T, the online
  // softmax, O^T += V^T . P^T.
  auto compute = [&](int buf, int kb) {
    if (kb > wave_max_pos) return;  // every key of the step is in the future of every row
    // some key of the step lies past some row's position (the causal diagonal, or
    // the tile's reach); uniform per wave, a scalar branch
    const bool need_mask = kb + kKeyStep - 1 > wave_min_pos;
    const _Float16 *K = lds + buf * L::kBufHalves;
    const _Float16 *V = K + L::kKHalves;
    f4_t s1[RB], s2[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      s1[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
      s2[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int cc = 4 * kk + g16;
      const u32x4 a1 = *reinterpret_cast<const u32x4 *>(K + key1 * D + ((cc ^ k_swizzle<D>(key1)) * 8));
      const u32x4 a2 = *reinterpret_cast<const u32x4 *>(K + key2 * D + ((cc ^ k_swizzle<D>(key2)) * 8));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        s1[rb] = mfma32<KV>(a1, qop[rb][kk], s1[rb]);
        s2[rb] = mfma32<KV>(a2, qop[rb][kk], s2[rb]);
      }
    }
    const float c = d.qk_scale;  // softmax scale * log2(e) (> 0); m is kept in these units
    u32x4 pk[RB], pl[RB];  // P^T operands: p (f16), or its hi and lo parts (bf16)
    bool rescale = false;
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = s1[rb][i];
        sc[4 + i] = s2[rb][i];
      }
      if (need_mask) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sc[j] = (kb + 8 * g16 + j <= row_pos[rb]) ? sc[j] : -INFINITY;
      }
      float mx = sc[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
      mx = max_xor_rows<16>(mx);
      mx = max_xor_rows<32>(mx);
      // Lazy rescale: the running max moves only when a score exceeds it by more
      // than kLazy (log2 units), so p = 2^(s*c - m) stays below 2^kLazy, well inside
      // the range of the 16-bit P operand and of the fp32 sums; the result does not
      // depend on m (numerator and denominator carry the same factor).
      const float mt = mx * c;
      const bool grow = mt > m[rb] + kLazy;
      const float mn = grow ? mt : m[rb];
      rescale |= grow;
      alpha[rb] = fast_exp2(m[rb] - mn);
      m[rb] = mn;
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = fast_exp2(__builtin_fmaf(sc[j], c, -mn));
      p_operands<KV>(p, pk[rb], pl[rb]);
    }
    if (__any(rescale)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        lsum[rb] *= alpha[rb];
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) o[rb][sl] *= alpha[rb];
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      lsum[rb] = mfma32<KV>(ones, pk[rb], lsum[rb]);
      if constexpr (kSplitP<KV>) lsum[rb] = mfma32<KV>(ones, pl[rb], lsum[rb]);
    }
    // V^T operand of slice sl, read one slice ahead of the products that use it
    auto vread = [&](int sl) {
      const int d0 = sl * 16 + vcol;
      const _Float16 *vp = V + vrow * D + ((d0 >> 3) ^ v_swizzle<D>(vrow)) * 8 + (d0 & 7);
      const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * D);
      return u32x4{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4 va[2];
    va[0] = vread(0);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl + 1 < NSL) va[(sl + 1) & 1] = vread(sl + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<KV>(va[sl & 1], pk[rb], o[rb][sl]);
      if constexpr (kSplitP<KV>) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<KV>(va[sl & 1], pl[rb], o[rb][sl]);
      }
    }
  };
  constexpr int NS = kStages;
  constexpr int U = NS % 2 ? 2 * NS : NS;  // unroll: stage ring and LDS buffer parity
  const int nsteps = (nkeys + kKeyStep - 1) / kKeyStep;
  Stage st[NS];
  StepBt bnext = bt_load(NS);  // clamped when the tile has fewer steps
#pragma unroll
  for (int i = 0; i < NS; ++i) gload(bt_load(i), st[i]);
  lstore(0, 0, st[0]);
  __syncthreads();
  // iteration n: read step n+NS+1's block-table entries, load step n+NS into the
  // stage step n used, compute step n from LDS, then move step n+1 (already in
  // registers) into the other LDS buffer.  Past the last step the loads repeat
  // the last block.
  auto iter = [&](int n, Stage &mine, const Stage &next) {
    const StepBt bn = bt_load(n + NS + 1);
    gload(bnext, mine);
    bnext = bn;
    compute(n & 1, n * kKeyStep);
    if (n + 1 < nsteps) lstore((n + 1) & 1, (n + 1) * kKeyStep, next);
    __syncthreads();
  };
  // Whole groups of U steps in an unguarded loop, then the (< U) remaining steps
  // once.  With a per-step guard inside the loop, its header gets several entries
  // and the compiler's wait counting, merging them, drains every load in flight
  // before each step issues its own: the ring would be one step deep instead of NS.
  int n0 = 0;
  for (; n0 + U <= nsteps; n0 += U) {
#pragma unroll
    for (int i = 0; i < U; ++i) iter(n0 + i, st[i % NS], st[(i + 1) % NS]);
  }
#pragma unroll
  for (int i = 0; i < U - 1; ++i)
    if (n0 + i < nsteps) iter(n0 + i, st[i % NS], st[(i + 1) % NS]);

  // ---- normalise and store: lane holds dims sl*16 + 4*g16 + i of query row c16 ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if (!row_ok[rb]) continue;
    const float inv = 1.f / lsum[rb][0];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out<KV>(d.out, row_out[rb] + sl * 16 + 4 * g16 + i, o[rb][sl][i] * inv);
  }
}

// Work list of prefill tiles, heaviest first over the whole step (longest
// processing time first: the tiles of a chunk with a long prior context start in
// the first round of workgroups, whichever chunk they belong to).  A tile's cost is
// its number of 32-key steps.  One workgroup of 256 threads: a counting sort of
// the tiles by cost (costs past kCostBuckets - 1 share the last bucket), in two
// passes over the sequences in rounds of 256.  Tiles of equal cost land in any
// order; each tile writes its own rows, so the order never changes a result.
constexpr int kCostBuckets = 1024;

__global__ __launch_bounds__(256) void pa_mixed_prep_kernel(MixedArgs a) {
  __shared__ int hist[kCostBuckets];
  __shared__ int part[256];
  const int tid = threadIdx.x;
  for (int b = tid; b < kCostBuckets; b += 256) hist[b] = 0;
  __syncthreads();
  // tiles of sequence s (0 for a decode row or a sequence past the batch), and
  // the cost bucket of its tile t
  auto tiles_of = [&](int s, int &first, int &ql) {
    if (s >= a.num_seqs) return 0;
    ql = a.qsl[s + 1] - a.qsl[s];
    if (ql <= 1) return 0;
    first = a.dec.ctx[s] - ql;
    return min((ql + a.qtok - 1) / a.qtok, (1 << kItemBits));
  };
  auto bucket = [&](int first, int ql, int t) {
    const int nkeys = first + min((t + 1) * a.qtok, ql);
    return min((nkeys + kKeyStep - 1) / kKeyStep, kCostBuckets - 1);
  };
  for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
    int first = 0, ql = 0;
    const int np = tiles_of(c0 + tid, first, ql);
    for (int t = 0; t < np; ++t) atomicAdd(&hist[bucket(first, ql, t)], 1);
  }
  __syncthreads();
  // start of every bucket in descending cost order: thread i owns buckets
  // B-1-4i .. B-4-4i (four in a row, highest first); scan the per-thread sums
  int loc[4], sum = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    loc[k] = hist[kCostBuckets - 1 - (4 * tid + k)];
    sum += loc[k];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    hist[kCostBuckets - 1 - (4 * tid + k)] = run;  // bucket start
    run += loc[k];
  }
  __syncthreads();
  for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
    const int s = c0 + tid;
    int first = 0, ql = 0;
    const int np = tiles_of(s, first, ql);
    for (int t = 0; t < np; ++t) {
      const int pos = atomicAdd(&hist[bucket(first, ql, t)], 1);
      if (pos < a.p_bound) a.p_items[pos] = (s << kItemBits) | t;
    }
  }
  if (tid == 0) a.hdr[0] = min(part[255], a.p_bound);
}

// Grid (Hkv, items): the kv head is the fastest index, so with workgroups handed to
// the 8 XCDs in turn, all tiles of one (sequence, kv head) run on one XCD (for
// 8 kv heads; on 8 / Hkv of them otherwise) and share its L2 copy of their K/V.
template <int KV, int D, int G>
__global__ __launch_bounds__(256) void pa_prefill_tiles_kernel(MixedArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[PrefillLds<D>::kBytes];
  const int x = blockIdx.y, h = blockIdx.x;
  if (x >= a.hdr[0]) return;
  const int item = a.p_items[x];
  prefill_tile<KV, D, G>(a, item >> kItemBits, h, item & ((1 << kItemBits) - 1), smem);
}

// ---- fallback for KV types without an MFMA tile path (fp32, fp8, int8): every
// query row runs the decode partition path with its own causal length ----
__device__ __forceinline__ void row_owner(const int32_t *qsl, const int32_t *seq_lens,
                                          int num_seqs, int t, int &s, int &n) {
  int lo = 0, hi = num_seqs;  // invariant: qsl[lo] <= t < qsl[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid;
  }
  s = lo;
  const int q_len = qsl[lo + 1] - qsl[lo];
  n = seq_lens[lo] - q_len + (t - qsl[lo]) + 1;
}

template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(kDecodeWaves *kWave) void pa_mixed_rows_kernel(MixedArgs a) {
  __shared__ float smem[decode_partition_smem_floats<D, G>()];
  const int t = blockIdx.z;
  int s, n;
  row_owner(a.qsl, a.dec.ctx, a.num_seqs, t, s, n);
  decode_partition<KV, QT, D, G>(a.dec, s, blockIdx.y, blockIdx.x, t, n, t, smem);
}

template <int QT, int D>
__global__ __launch_bounds__(D) void pa_mixed_rows_merge_kernel(MixedArgs a) {
  const int t = blockIdx.y;
  int s, n;
  row_owner(a.qsl, a.dec.ctx, a.num_seqs, t, s, n);
  merge_partitions<QT, D>(a.dec, t, blockIdx.x, threadIdx.x, n);
}

// ---------------------------------------------------------------------------------------
// host-side dispatch
// ---------------------------------------------------------------------------------------
template <int KV, int QT, int D, int G>
static hipError_t launch_tiles(const MixedArgs &a, bool stream_loads, hipStream_t st) {
  hipLaunchKernelGGL(pa_mixed_prep_kernel, dim3(1), dim3(256), 0, st, a);
  dim3 grid(a.dec.num_kv_heads, a.p_bound);
  hipLaunchKernelGGL((pa_prefill_tiles_kernel<KV, D, G>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_decode_stream(a.dec, KV, QT, D, G, a.num_seqs, stream_loads, st);
}

template <int KV, int QT, int D, int G>
static hipError_t launch_rows(const MixedArgs &a, int num_rows, hipStream_t st) {
  dim3 grid(a.dec.max_parts, a.dec.num_kv_heads, num_rows);
  hipLaunchKernelGGL((pa_mixed_rows_kernel<KV, QT, D, G>), grid, dim3(kDecodeWaves * kWave), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.dec.max_parts <= 1) return e;
  dim3 mg(a.dec.num_q_heads, num_rows);
  hipLaunchKernelGGL((pa_mixed_rows_merge_kernel<QT, D>), mg, dim3(D), 0, st, a);
  return hipGetLastError();
}

template <int KV, int QT, int D>
static hipError_t launch_g(const MixedArgs &a, int G, int num_rows, bool tiles, bool stream_loads,
                           hipStream_t st) {
  constexpr bool kMfma = (KV == PA_F16 || KV == PA_BF16);
#define PA_CASE(g)                                                              \
  case g:                                                                       \
    if constexpr (kMfma) {                                                      \
      if (tiles) return launch_tiles<KV, QT, D, g>(a, stream_loads, st);        \
    }                                                                           \
    return launch_rows<KV, QT, D, g>(a, num_rows, st);
  switch (G) {
    PA_CASE(1)
    PA_CASE(2)
    PA_CASE(4)
    PA_CASE(8)
  }
#undef PA_CASE
  return hipErrorInvalidValue;
}

template <int KV, int QT>
static hipError_t launch_d(const MixedArgs &a, int D, int G, int num_rows, bool tiles,
                           bool stream_loads, hipStream_t st) {
  if (D == 64) return launch_g<KV, QT, 64>(a, G, num_rows, tiles, stream_loads, st);
  if (D == 128) return launch_g<KV, QT, 128>(a, G, num_rows, tiles, stream_loads, st);
  return hipErrorInvalidValue;
}

bool mixed_uses_tiles(int kv_dtype) { return kv_dtype == PA_F16 || kv_dtype == PA_BF16; }

hipError_t launch_mixed(const MixedArgs &a, int kv_dtype, int q_dtype, int head_dim, int group,
                        int num_rows, bool stream_loads, hipStream_t st) {
  const bool tiles = mixed_uses_tiles(kv_dtype);
  switch (kv_dtype) {
    case PA_F32: return launch_d<PA_F32, PA_F32>(a, head_dim, group, num_rows, tiles, stream_loads, st);
    case PA_F16: return launch_d<PA_F16, PA_F16>(a, head_dim, group, num_rows, tiles, stream_loads, st);
    case PA_BF16: return launch_d<PA_BF16, PA_BF16>(a, head_dim, group, num_rows, tiles, stream_loads, st);
    case PA_FP8_E4M3:
      return q_dtype == PA_F16
                 ? launch_d<PA_FP8_E4M3, PA_F16>(a, head_dim, group, num_rows, tiles, stream_loads, st)
                 : launch_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, num_rows, tiles, stream_loads, st);
    case PA_I8:
      return q_dtype == PA_F16 ? launch_d<PA_I8, PA_F16>(a, head_dim, group, num_rows, tiles, stream_loads, st)
                               : launch_d<PA_I8, PA_BF16>(a, head_dim, group, num_rows, tiles, stream_loads, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
