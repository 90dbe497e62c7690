// Mixed continuous-batching step: chunked prefills and decodes in one launch.
//
// uml.org.cn "Continuous Batching": new requests' prefill work and running
// requests' decode steps share one batch.  5688vip chapter 3, section 3.1:
// generation is autoregressive, so query row i of a chunk that extends a
// sequence to seq_len tokens sits at position seq_len - q_len + i and attends to
// keys 0 .. that position.
//
// For f16 / bf16 and fp8 / int8 KV the step is two launches (after a small one that lists the
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
// 1-byte KV (fp8 E4M3FN, int8) runs the same tiles on its codes converted exactly to
// 16 bits in LDS (q's type for K, bf16 for V), with the scales folded into the score
// scale and the weights (see prefill_tile).  fp32 KV runs every query row through
// the partitioned decode path.
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
constexpr float kLazy = 8.f;    // running-max slack before a rescale (log2 units)

int mixed_tile_rows() { return kTileRows; }

template <int D, bool Q8>
struct PrefillLds {
  static constexpr int kKHalves = kKeyStep * D;     // K: [32 keys][D], chunks swizzled
  static constexpr int kVHalves = kKeyStep * D;     // V: [32 keys][D], chunks swizzled
  static constexpr int kBufHalves = kKHalves + kVHalves;
  // 16-bit K/V buffers.  16-bit pools load a step straight into its buffer two
  // iterations ahead (four: two in flight, the scored step, the deferred V).  1-byte
  // pools load codes into a ring of their own and convert a step into its buffer
  // one iteration ahead (three: converted, scored, deferred V).
  static constexpr int kBufs = Q8 ? 3 : 4;
  static constexpr int kCodeBytes = Q8 ? 2 * kKeyStep * D : 0;  // K + V codes of a step
  static constexpr int kCodeBufs = Q8 ? 2 : 0;
  static constexpr int kCodeOff = kBufs * kBufHalves * 2;       // bytes
  static constexpr int kBytes = kCodeOff + kCodeBufs * kCodeBytes;
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

// P^T operands of 4 probabilities (words 2*half and 2*half + 1) in the P.V MFMA's
// 16-bit type T.  The P.V product and the row sums see the same operands, so the
// output is sum(p~ v) / sum(p~) for the weights p~ as the MFMA inputs hold them.
//  f16: p rounded to nearest even (lo unused).  Each weight then carries a
//       relative error below 2^-11, which moves the output by less than 2^-11 of
//       the weighted spread |v - out| of the values -- the order of V's own f16
//       storage precision, and inside the f16 tolerance (a simulation of 25.6 M
//       outputs on unscaled N(0,1) data, few to hundreds of keys, peaked at 0.72
//       of the bar: max(2e-3, one ulp)).
//  bf16 pools (SPLIT): one rounding would be 2^-8 relative (3x the bar on such
//       data), so p is split into two parts, p ~= hi + lo: hi = p truncated to its
//       upper 16 bits (a byte permute of two values), lo = (p - hi) rounded to
//       nearest even, the difference exact in fp32; the pair holds p to 2^-15
//       relative and every product runs twice (hi, then lo).
//  1-byte pools: bf16, one rounding (2^-8 relative, within their 2e-2 tolerance).
template <int T, bool SPLIT>
__device__ __forceinline__ void p_operands_half(const float *p, u32x4 &hi, u32x4 &lo, int half) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float a = p[2 * i], b = p[2 * i + 1];
    if constexpr (!SPLIT) {
      if constexpr (T == PA_F16)
        hi[2 * half + i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, h2v_t));
      else
        hi[2 * half + i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{a, b}, b2v_t));
    } else {
      const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
      hi[2 * half + i] = __builtin_amdgcn_perm(ub, ua, 0x07060302u);  // upper halves of a, b
      const float ra = a - __builtin_bit_cast(float, ua & 0xFFFF0000u);
      const float rb = b - __builtin_bit_cast(float, ub & 0xFFFF0000u);
      lo[2 * half + i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2_t{ra, rb}, b2v_t));
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
// Pipeline, per 32-key step n: K/V of step n+2 go from HBM straight into LDS
// (LDS-DMA, no registers), the block-table entries of step n+3 are read, the scores
// and softmax of step n run beside the P.V product of step n-1 (whose V is still in
// LDS), and the wave waits for its loads of step n+1 before the barrier that hands
// them to every wave.  16-bit pools: the loads land in step n+2's 16-bit buffer.
// 1-byte pools (fp8 E4M3FN, int8): the codes land in a ring of code buffers, and
// each wave converts the rows it loaded itself -- exactly, to q's type for K and to
// bf16 for V -- into step n+1's 16-bit buffer once they have landed; the
// per-(block, kv head) scales are folded in afterwards: the key scale into each
// lane's score scale (a lane's 8 keys lie in one block), the value scale into the
// weights (p' = p * vs through the exponent), and the row sums are kept per lane in
// fp32 as sum(p' / vs).  Every load is issued unconditionally (indices clamped to the
// tile's last block) so the wait counts are fixed.  Each K or V operand read from
// LDS serves all RB row blocks of the wave.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void prefill_tile(const MixedArgs &a, int s, int h, int qt,
                                             char *smem) {
  constexpr bool Q8 = KV == PA_FP8_E4M3 || KV == PA_I8;
  static_assert(Q8 || KV == QT, "16-bit pools take queries of their own type");
  constexpr int MQ = QT;                     // QK MFMA type (q's type; K converted to it)
  constexpr int MP = Q8 ? PA_BF16 : KV;      // P.V MFMA type (V as stored, or codes as bf16)
  constexpr bool kSplit = KV == PA_BF16;     // P as hi + lo parts
  constexpr int RB = kRowBlocks;
  constexpr int QTOK = kTileRows / G;
  constexpr int NKK = D / 32;        // QK MFMAs along head_dim
  constexpr int NSL = D / 16;        // 16-dim output slices
  using L = PrefillLds<D, Q8>;
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

  // o: O^T slices.  lsum (16-bit pools): the running softmax denominators,
  // accumulated on the matrix cores as ones(16 x 32) . P^T (hi and lo parts for
  // bf16), so every element holds its query row's sum of the probabilities as the
  // P.V product used them.  lrow (1-byte pools): this lane's share of its row's sum
  // of the unscaled weights, in fp32.
  f4_t o[RB][NSL], lsum[RB];
  float m[RB], lrow[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    lrow[rb] = 0.f;
    lsum[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) o[rb][sl] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  constexpr uint32_t kOne2 = MP == PA_F16 ? 0x3C003C00u : 0x3F803F80u;  // two 16-bit 1.0s
  const u32x4 ones = u32x4{kOne2, kOne2, kOne2, kOne2};

  // ---- global -> LDS staging of one 32-key step (LDS-DMA) ----
  // gfx950's global_load_lds_dwordx4: each lane's 16 bytes land at m0 + 16 * lane
  // (checked on the MI355X), so a wave-wide load fills 1 KiB of LDS with no
  // registers in between.
  const char *kpool = reinterpret_cast<const char *>(d.k);
  const char *vpool = reinterpret_cast<const char *>(d.v);
  // 16-row tile indices of step n's two tiles (clamped to the last tile)
  struct StepBt {
    int64_t u0, u1;
  };
  const int sh = d.bs_shift;
  // The table row (and the scales) are read through the constant address space:
  // nothing writes them during the kernel, and these reads (uniform per wave) then
  // stay scalar loads -- the compiler would otherwise make vector loads of them after
  // the LDS-DMA statements below, which it cannot prove write no global memory, and a
  // wait for those would also wait for every load in flight.
  typedef const __attribute__((address_space(4))) int32_t *cint_p;
  typedef const __attribute__((address_space(4))) float *cfloat_p;
  const cint_p btc = (cint_p)(uintptr_t)bt;
  auto bt_load = [&](int n) {
    const int j0 = min(2 * n, nblk - 1), j1 = min(2 * n + 1, nblk - 1);
    StepBt r;
    r.u0 = tile_index(btc[j0 >> sh], Hkv, h, j0, sh);
    r.u1 = tile_index(btc[j1 >> sh], Hkv, h, j1, sh);
    return r;
  };
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  auto dma1 = [&](const char *gbase, uint32_t off, uint32_t lds_addr) {
    const uint64_t g = (uint64_t)(uintptr_t)gbase;
    const uint32_t glo = __builtin_amdgcn_readfirstlane((uint32_t)g);
    const uint32_t ghi = __builtin_amdgcn_readfirstlane((uint32_t)(g >> 32));
    const uint64_t gu = ((uint64_t)ghi << 32) | glo;
    const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds_addr);
    // No memory clobber: the compiler must keep its block-table reads scalar, which
    // it does only while no write to global memory may precede them.  The load's
    // LDS writes are ordered by the waits and barriers around it (both have side
    // effects, as this statement does, so none of them is moved across another).
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0v), "v"(off),
                 "s"(gu));
  };

  // 16-bit pools: a wave-wide load is RPW whole key rows; a lane picks the global
  // chunk whose swizzled position is its slot: chunk p ^ swizzle(key) of its key row
  // (the same row, so the wave's reads stay contiguous).  NL loads of K and NL of V
  // per wave and step.
  constexpr int CPR = D / 8;                    // 16-byte chunks per key row
  constexpr int RPW = 64 / CPR;                 // key rows per wave-wide load
  constexpr int NL = Q8 ? 0 : kKeyStep / RPW / 4;
  // 1-byte pools: the step's K and V codes are D/16 wave-wide loads, K first; wave w
  // issues QPW of them (K for half the waves, V for the other half), each 1 KiB =
  // RPQ key rows, the lane's 16 codes being chunk p of row r.
  constexpr int QPW = Q8 ? D / 64 : 0;
  constexpr int RPQ = 1024 / D;                 // key rows per code load
  constexpr int CPQ = D / 16;                   // 16-code chunks per key row
  constexpr int KLD = D / 32;                   // code loads of K per step
  constexpr int LPW = Q8 ? QPW : 2 * NL;        // loads per wave and step
  uint32_t koff[Q8 ? 1 : NL], voff[Q8 ? 1 : NL];  // 16-bit: the lane's chunk in its tile
  uint32_t qoff[Q8 ? QPW : 1];                    // 1-byte: the lane's code chunk in its tile
  if constexpr (!Q8) {
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int key = (wave * NL + j) * RPW + lane / CPR, p = lane % CPR;
      koff[j] = (uint32_t)((key % kBlock) * D * 2 + (p ^ k_swizzle<D>(key)) * 16);
      voff[j] = (uint32_t)((key % kBlock) * D * 2 + (p ^ v_swizzle<D>(key)) * 16);
    }
  } else {
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int lw = wave * QPW + j;
      const int r = (lw % KLD) * RPQ + lane / CPQ, p = lane % CPQ;
      qoff[j] = (uint32_t)((r % kBlock) * D + p * 16);
    }
  }
  // the step's K and V tiles: into 16-bit buffer bi, or (1-byte) into code buffer bi
  auto dma_step = [&](const StepBt &b, int bi) {
    if constexpr (!Q8) {
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int lw = wave * NL + j;                // this load's 1 KiB of the tile pair
        const int64_t tile = ((lw * RPW) / kBlock ? b.u1 : b.u0) * (int64_t)(kBlock * D * 2);
        const uint32_t at = lds_base + (uint32_t)((bi * L::kBufHalves) * 2 + lw * 1024);
        dma1(kpool + tile, koff[j], at);
        dma1(vpool + tile, voff[j], at + L::kKHalves * 2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        const int lw = wave * QPW + j;
        const int64_t tile = (((lw % KLD) * RPQ) / kBlock ? b.u1 : b.u0) * (int64_t)(kBlock * D);
        const uint32_t at = lds_base + (uint32_t)(L::kCodeOff + bi * L::kCodeBytes + lw * 1024);
        dma1((lw < KLD ? kpool : vpool) + tile, qoff[j], at);
      }
    }
  };
  // s_waitcnt vmcnt(c) (the other counters left alone): the loads this wave issued,
  // all but the newest c, have landed in LDS.  The library code in the step loop
  // issues no other vector-memory instruction, so the count is exact.
  auto wait_loads = [&](auto c) {
    constexpr int n = decltype(c)::value;
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
  };
  // 16-bit pools: V rows of step n at or past nkeys (the tile's reach; they may hold
  // anything, NaN included) are zeroed after this wave's own loads of them have
  // landed: their weights are zero, and 0 * NaN would not be.  K needs no fix: those
  // keys are masked by selection.  The store is written out with its waits (all
  // loads, then the store itself) so that the compiler, which does not see the
  // loads, cannot place it before them.  Only the step that reaches past nkeys takes
  // this path.
  auto fix_tail = [&](int n, int bi) {
    const int kb = n * kKeyStep;
    if (kb + kKeyStep <= nkeys) return;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int lw = wave * NL + j;
      const int key = lw * RPW + lane / CPR;
      const uint32_t at = lds_base + (uint32_t)((bi * L::kBufHalves + L::kKHalves) * 2 + lw * 1024 +
                                                lane * 16);
      const u32x4 z = u32x4{0, 0, 0, 0};
      if (kb + key >= nkeys)
        asm volatile("s_waitcnt vmcnt(0)\n\tds_write_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(at),
                     "v"(z));
    }
  };
  // 1-byte pools: after this wave's code loads of step n have landed (the caller
  // waits), its lanes convert their own 16 codes each into step n's 16-bit buffer bi
  // (K in q's type, V in bf16; both exact), in the same swizzled layout the 16-bit
  // pools load; rows at or past nkeys become zeros.  The read of the codes is written
  // out with its wait, so the compiler (which does not see the loads) keeps it after
  // the wait for them.
  auto convert_step = [&](int n, int bi, int ci) {
    const int kb = n * kKeyStep;
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int lw = wave * QPW + j;
      const bool is_k = lw < KLD;
      const int r = (lw % KLD) * RPQ + lane / CPQ, p = lane % CPQ;
      const uint32_t at = lds_base + (uint32_t)(L::kCodeOff + ci * L::kCodeBytes + lw * 1024 + lane * 16);
      u32x4 c;
      asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(c) : "v"(at));
      uint32_t w[8];
      if (is_k) {  // uniform per load
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[2 * e] = codes2_to_16<KV, MQ, false>(c[e]);
          w[2 * e + 1] = codes2_to_16<KV, MQ, true>(c[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[2 * e] = codes2_to_16<KV, PA_BF16, false>(c[e]);
          w[2 * e + 1] = codes2_to_16<KV, PA_BF16, true>(c[e]);
        }
      }
      if (kb + r >= nkeys) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = 0u;
      }
      _Float16 *dst = lds + bi * L::kBufHalves + (is_k ? 0 : L::kKHalves) + r * D;
      const int sw = is_k ? k_swizzle<D>(r) : v_swizzle<D>(r);
      *reinterpret_cast<u32x4 *>(dst + ((2 * p) ^ sw) * 8) = u32x4{w[0], w[1], w[2], w[3]};
      *reinterpret_cast<u32x4 *>(dst + ((2 * p + 1) ^ sw) * 8) = u32x4{w[4], w[5], w[6], w[7]};
    }
  };
  // 1-byte pools: the step's key and value scales (per tile), for the lane's keys
  struct StepScale {
    float k0, k1, v0, v1;
  };
  const cfloat_p ksc = (cfloat_p)(uintptr_t)d.k_scale;
  const cfloat_p vsc = (cfloat_p)(uintptr_t)d.v_scale;
  auto scale_load = [&](const StepBt &b) {
    StepScale r{1.f, 1.f, 1.f, 1.f};
    if constexpr (Q8) {
      r.k0 = ksc[b.u0 >> sh];
      r.k1 = ksc[b.u1 >> sh];
      r.v0 = vsc[b.u0 >> sh];
      r.v1 = vsc[b.u1 >> sh];
    }
    return r;
  };

  const int key1 = 8 * (c16 >> 2) + (c16 & 3);  // key row of this lane in QK product 1
  const int key2 = key1 + 4;                      // ... in product 2
  // V^T operand of slice sl: this lane reads dims 16 sl + vcol .. +3 of key rows
  // vrow (keys 8 g16 .. +3 of the operand) and vrow + 4 (keys + 4 .. +7); the
  // transposed read returns dim 16 sl + c16 of the 4 keys.  vrow + 4 shares vrow's
  // swizzle (bit 2 of the key is not in it).
  const int vrow = 8 * g16 + (c16 >> 2), vcol = 4 * (c16 & 3);
  // 16-bit buffer of the step with index i modulo the unroll (i >= -1; i = -1 at step
  // 0 is the zeroed V that the first step's deferred product reads); the unroll is a
  // multiple of kBufs, so i modulo kBufs is the step's buffer
  auto buf_of = [&](int i) { return lds + ((i + L::kBufs) % L::kBufs) * L::kBufHalves; };
  // P^T operands of the step whose P.V product is still to run (deferred by one
  // step), zero before the first
  u32x4 pp[RB], ppl[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    pp[rb] = u32x4{0, 0, 0, 0};
    ppl[rb] = u32x4{0, 0, 0, 0};
  }
  auto vread_from = [&](const _Float16 *Vb, int sl) {
    const int d0 = sl * 16 + vcol;
    const _Float16 *vp = Vb + vrow * D + ((d0 >> 3) ^ v_swizzle<D>(vrow)) * 8 + (d0 & 7);
    const u32x2 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * D);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
  };
  // O^T += V^T . P^T and (16-bit pools) the row sums for the held P^T operands, V
  // from buffer Vb
  auto pv_product = [&](const _Float16 *Vb) {
    if constexpr (!Q8) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        lsum[rb] = mfma32<MP>(ones, pp[rb], lsum[rb]);
        if constexpr (kSplit) lsum[rb] = mfma32<MP>(ones, ppl[rb], lsum[rb]);
      }
    }
    // V^T operand of slice sl, read one slice ahead of the products that use it
    u32x4 va[2];
    va[0] = vread_from(Vb, 0);
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      if (sl + 1 < NSL) va[(sl + 1) & 1] = vread_from(Vb, sl + 1);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<MP>(va[sl & 1], pp[rb], o[rb][sl]);
      if constexpr (kSplit) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<MP>(va[sl & 1], ppl[rb], o[rb][sl]);
      }
    }
  };
  // Step n (keys kb ..; i = n modulo the unroll, sc = its scales): S^T = K . Q^T and
  // the online softmax of step n, and the P.V product of step n-1.  The two are
  // independent, so the softmax's VALU work and the previous step's MFMAs can
  // interleave; the rescale of the accumulators by step n's factor follows the
  // product of step n-1 (whose P was relative to the old maximum).
  auto full_step = [&](int i, int kb, const StepScale &sc) {
    // some key of the step lies past some row's position (the causal diagonal, or
    // the tile's reach); uniform per wave, a scalar branch
    const bool need_mask = kb + kKeyStep - 1 > wave_min_pos;
    const _Float16 *K = buf_of(i);
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
        s1[rb] = mfma32<MQ>(a1, qop[rb][kk], s1[rb]);
        s2[rb] = mfma32<MQ>(a2, qop[rb][kk], s2[rb]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // the score products stay ahead of the block below
    if (need_mask) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const bool vis = kb + 8 * g16 + j <= row_pos[rb];
          if (j < 4) s1[rb][j] = vis ? s1[rb][j] : -INFINITY;
          else s2[rb][j - 4] = vis ? s2[rb][j - 4] : -INFINITY;
        }
    }
    // Score scale of this lane's keys (softmax scale * log2(e), > 0; m is kept in
    // these units), for 1-byte pools times the key scale of their block.  The value
    // scale enters the weights through the exponent: p' = 2^(s*c - m + log2 vs).  A
    // zero scale (an all-zero tile) is taken as 1e-30: its codes give zero scores and
    // values either way, and the weights stay finite.
    float c = d.qk_scale, lvs = 0.f, ivs = 1.f;
    if constexpr (Q8) {
      const bool hi = g16 >= 2;  // keys 8*g16 .. +7 lie in the step's second block
      c *= fmaxf(hi ? sc.k1 : sc.k0, 1e-30f);
      const float vs = fmaxf(hi ? sc.v1 : sc.v0, 1e-30f);
      lvs = __builtin_amdgcn_logf(vs);
      ivs = __builtin_amdgcn_rcpf(vs);
    }
    // The softmax of step n and the P.V product of step n-1 (independent) run as
    // NSL + 1 phases, each holding a share of both: the product's MFMAs of one V
    // slice (the row sums first) and a piece of the softmax's VALU work, the V
    // reads two phases ahead of their products.  A scheduling fence closes each
    // phase, so the compiler cannot regroup the MFMAs into one run and the VALU work
    // into another: inside a phase the matrix cores run the MFMAs while the vector
    // unit works through its piece.
    u32x4 pn[RB], pnl[RB];  // P^T operands of step n (and lo parts for bf16 pools)
    bool rescale = false;
    float alpha[RB], mx[RB], mnew[RB];
    // 1-byte pools: this lane's sum of step n's weights (relative to the new max);
    // added to lrow only after lrow has been rescaled to that max
    float lstep[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) lstep[rb] = 0.f;
    // softmax pieces in order: local maxima (one per row block), the cross-lane max
    // and the running-max update (one per row block), then the weights and their
    // operands a half (4 keys) at a time
    constexpr int kPieces = 4 * RB;
    auto softmax_piece = [&](int k) {
      if (k < RB) {
        const int rb = k;
        const float v = max3_raw(max3_raw(s1[rb][0], s1[rb][1], s1[rb][2]),
                                 max3_raw(s1[rb][3], s2[rb][0], s2[rb][1]),
                                 max_raw(s2[rb][2], s2[rb][3]));
        mx[rb] = v * c;  // c > 0 keeps the order
      } else if (k < 2 * RB) {
        const int rb = k - RB;
        // Lazy rescale: the running max moves only when a score exceeds it by more
        // than kLazy (log2 units), so p = 2^(s*c - m) stays below 2^kLazy, well
        // inside the range of the 16-bit P operand and of the fp32 sums; the result
        // does not depend on m (numerator and denominator carry the same factor).
        const float mt = max_xor_rows<32>(max_xor_rows<16>(mx[rb]));
        const bool grow = mt > m[rb] + kLazy;
        mnew[rb] = grow ? mt : m[rb];
        rescale |= grow;
        alpha[rb] = m[rb] - mnew[rb];  // log2 of the rescale factor, 0 when the max stays
        m[rb] = mnew[rb];
      } else {
        const int rb = (k - 2 * RB) >> 1, half = (k - 2 * RB) & 1;
        const f4_t &sv = half ? s2[rb] : s1[rb];
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = fast_exp2(__builtin_fmaf(sv[j], c, lvs - mnew[rb]));
        if constexpr (Q8) lstep[rb] = __builtin_fmaf((p[0] + p[1]) + (p[2] + p[3]), ivs, lstep[rb]);
        p_operands_half<MP, kSplit>(p, pn[rb], pnl[rb], half);
        // The operands are used only by the next step's product; without a use
        // here the compiler sinks their computation there, out of this phase.
        asm volatile("" ::"v"(pn[rb][2 * half]), "v"(pn[rb][2 * half + 1]));
        if constexpr (kSplit)
          asm volatile("" ::"v"(pnl[rb][2 * half]), "v"(pnl[rb][2 * half + 1]));
      }
    };
    const _Float16 *Vb = buf_of(i - 1) + L::kKHalves;  // step n-1's V
    constexpr int NPH = NSL + 1;
    u32x4 va[3];
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      if (ph == 0) {
        va[0] = vread_from(Vb, 0);
        if (NSL > 1) va[1] = vread_from(Vb, 1);
      } else if (ph + 1 < NSL) {
        va[(ph + 1) % 3] = vread_from(Vb, ph + 1);
      }
      if (ph == 0) {
        if constexpr (!Q8) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            lsum[rb] = mfma32<MP>(ones, pp[rb], lsum[rb]);
            if constexpr (kSplit) lsum[rb] = mfma32<MP>(ones, ppl[rb], lsum[rb]);
          }
        }
      } else {
        const int sl = ph - 1;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<MP>(va[sl % 3], pp[rb], o[rb][sl]);
        if constexpr (kSplit) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<MP>(va[sl % 3], ppl[rb], o[rb][sl]);
        }
      }
#pragma unroll
      for (int k = 0; k < kPieces; ++k)
        if (k * NPH / kPieces == ph) softmax_piece(k);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (__any(rescale)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float f = fast_exp2(alpha[rb]);
        lsum[rb] *= f;
        lrow[rb] *= f;
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) o[rb][sl] *= f;
      }
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (Q8) lrow[rb] += lstep[rb];
      pp[rb] = pn[rb];
      ppl[rb] = pnl[rb];
    }
  };

  constexpr int kAhead = 2;  // a step's loads go out this many iterations before its scores
  // unroll: a multiple of every ring (16-bit buffers, code buffers, scales), so every
  // unrolled step's slots are compile-time
  constexpr int U = Q8 ? 6 : L::kBufs;
  static_assert(U % L::kBufs == 0 && U % (Q8 ? L::kCodeBufs : 1) == 0, "unroll cycles the rings");
  static_assert(Q8 ? L::kBufs >= 3 : kAhead + 2 <= L::kBufs, "buffers of the steps in use");
  constexpr int kScaleRing = Q8 ? kAhead + 1 : 1;  // 1-byte pools: scales of steps n .. n+kAhead
  constexpr int kCB = Q8 ? L::kCodeBufs : 1;       // code buffers (none for 16-bit pools)
  static_assert(U % kScaleRing == 0, "unroll cycles the scale ring");
  const int nsteps = (nkeys + kKeyStep - 1) / kKeyStep;
  // this wave's loads of kAhead - 1 steps: what may still be in flight when a step's
  // loads must have landed
  using AheadLess1 = std::integral_constant<int, LPW * (kAhead - 1)>;
  // The q operands have landed before the first LDS-DMA load is issued: the
  // compiler's own waits for them would otherwise sit inside the step loop and,
  // counting loads it cannot see, drain the prefetch every time round.
  wait_loads(std::integral_constant<int, 0>{});
  {  // the V that step 0's deferred product (with P = 0) reads: zeros, never NaN
    _Float16 *Vz = buf_of(-1) + L::kKHalves;
#pragma unroll
    for (int c = tid; c < L::kVHalves / 8; c += 256)
      *reinterpret_cast<u32x4 *>(Vz + 8 * c) = u32x4{0, 0, 0, 0};
  }
  StepScale scl[kScaleRing];
#pragma unroll
  for (int i = 0; i < kAhead; ++i) {  // clamped past the last step
    const StepBt b = bt_load(i);
    dma_step(b, Q8 ? i % kCB : i);
    scl[i] = scale_load(b);
  }
  StepBt bnext = bt_load(kAhead);
  wait_loads(AheadLess1{});
  if constexpr (Q8)
    convert_step(0, 0, 0);
  else
    fix_tail(0, 0);
  __syncthreads();
  // iteration n (i = n mod U): issue step n+kAhead's loads (and read its scales),
  // read the block-table entries of the step after, run step n (with the product of
  // step n-1), then wait for step n+1's loads (and convert them, for 1-byte pools).
  // A wave whose rows end before the tile's last step runs its remaining steps fully
  // masked (zero weights): it would otherwise wait at the barriers, and one code path
  // keeps its registers within two waves per SIMD.  Past the last step the loads
  // repeat the last block into free buffers.
  auto iter = [&](int n, int i) {
    dma_step(bnext, Q8 ? (i + kAhead) % kCB : (i + kAhead) % L::kBufs);
    scl[(i + kAhead) % kScaleRing] = scale_load(bnext);
    bnext = bt_load(n + kAhead + 1);
    full_step(i, n * kKeyStep, scl[i % kScaleRing]);
    wait_loads(AheadLess1{});  // step n+1's loads have landed; step n+2's may be in flight
    if (n + 1 < nsteps) {
      if constexpr (Q8)
        convert_step(n + 1, (i + 1) % L::kBufs, (i + 1) % kCB);
      else
        fix_tail(n + 1, (i + 1) % L::kBufs);
    }
    __syncthreads();
  };
  int n0 = 0;
  for (; n0 + U <= nsteps; n0 += U) {
#pragma unroll
    for (int i = 0; i < U; ++i) iter(n0 + i, i);
  }
#pragma unroll
  for (int i = 0; i < U - 1; ++i)
    if (n0 + i < nsteps) iter(n0 + i, i);
  pv_product(lds + ((nsteps - 1) % L::kBufs) * L::kBufHalves + L::kKHalves);  // the last product
  // no load may still be writing this workgroup's LDS when it exits
  wait_loads(std::integral_constant<int, 0>{});

  // ---- normalise and store: lane holds dims sl*16 + 4*g16 + i of query row c16 ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float l;
    if constexpr (Q8) {  // the row's sum over its four lanes (g16 = 0 .. 3)
      l = lrow[rb];
      l += __shfl_xor(l, 16, 64);
      l += __shfl_xor(l, 32, 64);
    } else {
      l = lsum[rb][0];
    }
    if (!row_ok[rb]) continue;
    const float inv = 1.f / l;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out<QT>(d.out, row_out[rb] + sl * 16 + 4 * g16 + i, o[rb][sl][i] * inv);
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
template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(256) void pa_prefill_tiles_kernel(MixedArgs a) {
  __shared__ __attribute__((aligned(16)))
  char smem[PrefillLds<D, KV == PA_FP8_E4M3 || KV == PA_I8>::kBytes];
  const int x = blockIdx.y, h = blockIdx.x;
  if (x >= a.hdr[0]) return;
  const int item = a.p_items[x];
  prefill_tile<KV, QT, D, G>(a, item >> kItemBits, h, item & ((1 << kItemBits) - 1), smem);
}

// ---- fp32 KV (no MFMA tile path): every query row runs the decode partition path
// with its own causal length ----
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
  hipLaunchKernelGGL((pa_prefill_tiles_kernel<KV, QT, D, G>), grid, dim3(256), 0, st, a);
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
  constexpr bool kMfma = KV != PA_F32;  // MFMA prefill tiles: 16-bit and 1-byte pools
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

bool mixed_uses_tiles(int kv_dtype) {
  return kv_dtype == PA_F16 || kv_dtype == PA_BF16 || kv_dtype == PA_FP8_E4M3 || kv_dtype == PA_I8;
}

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
