// Mixed continuous-batching step: chunked prefills and decodes in one launch.
//
// uml.org.cn "Continuous Batching": new requests' prefill work and running
// requests' decode steps share one batch.  5688vip chapter 3, section 3.1:
// generation is autoregressive, so query row i of a chunk that extends a
// sequence to seq_len tokens sits at position seq_len - q_len + i and attends to
// keys 0 .. that position.
//
// One launch runs two kinds of workgroups, from a work list built on the device:
//  * prefill tiles (f16 / bf16 KV): 128 query rows -- (token, head) pairs of one
//    kv head's GQA group -- against 32-key steps of the chunk's context, with the
//    dense products on MFMA (v_mfma_f32_16x16x32_{f16,bf16}):
//      S^T = K . Q^T   (A = 16 keys x 32 dims from LDS, B = q rows in registers)
//      O^T += V^T . P^T (A = 16 dims x 32 keys of the transposed V tile in LDS,
//                        B = the probabilities straight from S^T's registers)
//    The two QK products of a step take their 16 key rows in an interleaved order
//    (first: keys 8(r/4) + r%4, second: the same + 4) so that each lane's 8 scores
//    are the 8 consecutive keys its P^T operand needs; computing O^T rather than O
//    keeps each query row's running max, sum and rescale inside one lane.
//  * decode rows (q_len == 1): the partitioned VALU decode path of decode_impl.h.
// Decode rows split over several partitions are combined by a second launch.
#include "decode_impl.h"

namespace pa {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kRowBlocks = 1;   // 16-row MFMA blocks per wave
constexpr int kTileRows = 4 * 16 * kRowBlocks;  // query rows (token, head) per prefill workgroup
constexpr int kKeyStep = 32;    // keys per step (two blocks)
constexpr int kVtStride = 40;   // halves per transposed-V row: 32 keys + 8 pad (80 bytes)
constexpr int kBtCache = 512;   // block-table entries of a tile kept in LDS (8192 keys)
constexpr int kItemBits = 12;   // item = (sequence << 12) | tile or partition index


template <int D>
struct PrefillLds {
  static constexpr int kKHalves = kKeyStep * D;     // K: [32 keys][D], chunks swizzled
  static constexpr int kVtHalves = D * kVtStride;   // V^T: [D][32 keys + pad], groups swizzled
  static constexpr int kBufHalves = kKHalves + kVtHalves;
  static constexpr int kBtOffset = 2 * kBufHalves * 2;        // bytes: two K/V buffers first
  static constexpr int kBytes = kBtOffset + kBtCache * 4;     // then the block-table cache
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

// Round 8 floats to the MFMA input type and pack them (nearest even).
template <int KV>
__device__ __forceinline__ u32x4 pack8(const float *p) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t lo, hi;
    if constexpr (KV == PA_F16) {
      lo = __builtin_bit_cast(uint16_t, (_Float16)p[2 * i]);
      hi = __builtin_bit_cast(uint16_t, (_Float16)p[2 * i + 1]);
    } else {
      lo = __builtin_bit_cast(uint16_t, (__bf16)p[2 * i]);
      hi = __builtin_bit_cast(uint16_t, (__bf16)p[2 * i + 1]);
    }
    r[i] = lo | (hi << 16);
  }
  return r;
}

// One prefill tile: query tokens [qt*QTOK, ...) of sequence s, kv head h.
// Rows: wave w, row block rb, lane column c16 -> row (w*RB + rb)*16 + c16 = token*G + head.
// Pipeline: the block-table entries of the tile sit in LDS; K/V of step n+2 are
// loaded into registers while step n is computed from LDS and step n+1 is written
// to the other LDS buffer.
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
  int32_t *bt_lds = reinterpret_cast<int32_t *>(smem + L::kBtOffset);
  const DecodeArgs &d = a.dec;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g16 = lane >> 4, c16 = lane & 15;
  const int q0 = a.qsl[s], q_len = a.qsl[s + 1] - q0;
  const int first_pos = d.ctx[s] - q_len;
  const int t0 = qt * QTOK;
  const int t_end = min(t0 + QTOK, q_len);
  const int nkeys = first_pos + t_end;  // keys any row of the tile can see
  const int min_pos = first_pos + t0;
  const int32_t *bt = d.bt + (int64_t)s * d.max_blocks_per_seq;
  const int Hq = d.num_q_heads, Hkv = d.num_kv_heads;

  // block-table entries of the tile's keys -> LDS (beyond the cache: read directly)
  const int nblk = (nkeys + kBlock - 1) / kBlock;
  for (int i = tid; i < nblk && i < kBtCache; i += 256) bt_lds[i] = bt[i];

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

  f4_t o[RB][NSL];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegBig;
    l[rb] = 0.f;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) o[rb][sl] = f4_t{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // block-table cache ready

  // ---- global -> registers -> LDS staging of one 32-key step ----
  const char *kpool = reinterpret_cast<const char *>(d.k);
  const char *vpool = reinterpret_cast<const char *>(d.v);
  struct Stage {
    u32x4 k[NCH], v[NCH];
  };
  auto gload = [&](int kb, Stage &st) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + 256 * c;
      const int key = q / CPR, cc = q % CPR;
      const int kabs = kb + key;
      if (kabs < nkeys) {  // keys past the tile's reach are never read (zeros instead)
        const int bi = kabs / kBlock;
        const int64_t tile = (int64_t)(bi < kBtCache ? bt_lds[bi] : bt[bi]) * Hkv + h;
        const int64_t off = (tile * kBlock + (kabs % kBlock)) * D * 2 + cc * 16;
        st.k[c] = *reinterpret_cast<const u32x4 *>(kpool + off);
        st.v[c] = *reinterpret_cast<const u32x4 *>(vpool + off);
      } else {
        st.k[c] = u32x4{0, 0, 0, 0};
        st.v[c] = u32x4{0, 0, 0, 0};
      }
    }
  };
  // V^T rows hold the 32 keys in 4 groups of 8; group gk of dim row d sits at
  // position gk ^ ((d / 8) & 3) so that a wave's 2-byte stores spread over banks.
  auto lstore = [&](int buf, const Stage &st) {
    _Float16 *K = lds + buf * L::kBufHalves;
    uint16_t *Vt = reinterpret_cast<uint16_t *>(K + L::kKHalves);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int q = tid + 256 * c;
      const int key = q / CPR, cc = q % CPR;
      const int pc = cc ^ (key & (CPR - 1));  // swizzle: rows hit different banks
      *reinterpret_cast<u32x4 *>(K + key * D + pc * 8) = st.k[c];
      const int col = ((key >> 3) ^ (cc & 3)) * 8 + (key & 7);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        Vt[(cc * 8 + 2 * w) * kVtStride + col] = (uint16_t)(st.v[c][w] & 0xffffu);
        Vt[(cc * 8 + 2 * w + 1) * kVtStride + col] = (uint16_t)(st.v[c][w] >> 16);
      }
    }
  };

  const int key1 = 8 * (c16 >> 2) + (c16 & 3);  // key row of this lane in QK product 1
  const int key2 = key1 + 4;                      // ... in product 2
  auto compute = [&](int buf, int kb) {
    const _Float16 *K = lds + buf * L::kBufHalves;
    const _Float16 *Vt = K + L::kKHalves;
    f4_t s1[RB], s2[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      s1[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
      s2[rb] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int cc = 4 * kk + g16;
      const u32x4 a1 = *reinterpret_cast<const u32x4 *>(K + key1 * D + ((cc ^ (key1 & (CPR - 1))) * 8));
      const u32x4 a2 = *reinterpret_cast<const u32x4 *>(K + key2 * D + ((cc ^ (key2 & (CPR - 1))) * 8));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        s1[rb] = mfma32<KV>(a1, qop[rb][kk], s1[rb]);
        s2[rb] = mfma32<KV>(a2, qop[rb][kk], s2[rb]);
      }
    }
    const bool need_mask = kb + kKeyStep - 1 > min_pos;
    u32x4 pk[RB];
    bool rescale = false;
    float alpha[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = s1[rb][i] * d.qk_scale;
        sc[4 + i] = s2[rb][i] * d.qk_scale;
      }
      if (need_mask) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sc[j] = (kb + 8 * g16 + j <= row_pos[rb]) ? sc[j] : kNegBig;
      }
      float mx = sc[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) mx = fmaxf(mx, sc[j]);
      mx = fmaxf(mx, xor_lanes<16>(mx));
      mx = fmaxf(mx, xor_lanes<32>(mx));
      const float mn = fmaxf(m[rb], mx);
      rescale |= mn > m[rb];
      alpha[rb] = fast_exp2(m[rb] - mn);
      m[rb] = mn;
      float p[8], ps = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(sc[j] - mn);
        ps += p[j];
      }
      l[rb] = l[rb] * alpha[rb] + ps;
      pk[rb] = pack8<KV>(p);
    }
    if (__any(rescale)) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int sl = 0; sl < NSL; ++sl) o[rb][sl] *= alpha[rb];
    }
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      const int dim = sl * 16 + c16;
      const u32x4 va = *reinterpret_cast<const u32x4 *>(
          Vt + dim * kVtStride + ((g16 ^ ((dim >> 3) & 3)) * 8));
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[rb][sl] = mfma32<KV>(va, pk[rb], o[rb][sl]);
    }
  };

  const int nsteps = (nkeys + kKeyStep - 1) / kKeyStep;
  Stage sa, sb;
  gload(0, sa);
  if (nsteps > 1) gload(kKeyStep, sb);
  lstore(0, sa);
  __syncthreads();
  // iteration n: load step n+2 into the stage step n used, compute step n from LDS,
  // then move step n+1 (already in registers) into the other LDS buffer.
  auto iter = [&](int n, Stage &mine, Stage &next) {
    if (n + 2 < nsteps) gload((n + 2) * kKeyStep, mine);
    compute(n & 1, n * kKeyStep);
    if (n + 1 < nsteps) lstore((n + 1) & 1, next);
    __syncthreads();
  };
  for (int n = 0; n < nsteps; n += 2) {
    iter(n, sa, sb);
    if (n + 1 < nsteps) iter(n + 1, sb, sa);
  }

  // ---- normalise and store: lane holds dims sl*16 + 4*g16 + i of query row c16 ----
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float tot = l[rb];
    tot += xor_lanes<16>(tot);
    tot += xor_lanes<32>(tot);
    if (!row_ok[rb]) continue;
    const float inv = 1.f / tot;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        store_out<KV>(d.out, row_out[rb] + sl * 16 + 4 * g16 + i, o[rb][sl][i] * inv);
  }
}

template <int D, int G>
constexpr int mixed_lds_bytes() {
  constexpr int a = PrefillLds<D>::kBytes;
  constexpr int b = decode_partition_smem_floats<D, G>() * 4;
  return a > b ? a : b;
}

// Work list: prefill tiles (heaviest tile of each chunk first), then decode
// partitions.  One workgroup of 256 threads scans the sequences in rounds of 256.
__global__ __launch_bounds__(256) void pa_mixed_prep_kernel(MixedArgs a) {
  __shared__ int sp[256], sd[256];
  const int tid = threadIdx.x;
  const int part_tokens = a.dec.part_blocks * kBlock;
  int base_p = 0, base_d = 0;
  for (int c0 = 0; c0 < a.num_seqs; c0 += 256) {
    const int s = c0 + tid;
    int np = 0, nd = 0;
    if (s < a.num_seqs) {
      const int ql = a.qsl[s + 1] - a.qsl[s];
      if (ql > 1) {
        np = min((ql + a.qtok - 1) / a.qtok, (1 << kItemBits));
      } else {
        const int n = a.dec.ctx[s];
        nd = n > 0 ? min((n + part_tokens - 1) / part_tokens, a.dec.max_parts) : 1;
      }
    }
    sp[tid] = np;
    sd[tid] = nd;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {  // inclusive scans
      const int vp = tid >= off ? sp[tid - off] : 0;
      const int vd = tid >= off ? sd[tid - off] : 0;
      __syncthreads();
      sp[tid] += vp;
      sd[tid] += vd;
      __syncthreads();
    }
    const int ep = base_p + sp[tid] - np, ed = base_d + sd[tid] - nd;
    for (int k = 0; k < np && ep + k < a.p_bound; ++k)
      a.p_items[ep + k] = (s << kItemBits) | (np - 1 - k);
    for (int k = 0; k < nd && ed + k < a.d_bound; ++k) a.d_items[ed + k] = (s << kItemBits) | k;
    base_p += sp[255];
    base_d += sd[255];
    __syncthreads();
  }
  if (tid == 0) {
    a.hdr[0] = min(base_p, a.p_bound);
    a.hdr[1] = min(base_d, a.d_bound);
  }
}

template <int KV, int QT, int D, int G>
__global__ __launch_bounds__(256) void pa_mixed_kernel(MixedArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[mixed_lds_bytes<D, G>()];
  const int x = blockIdx.x, h = blockIdx.y;
  if (x < a.p_bound) {
    if (x >= a.hdr[0]) return;
    const int item = a.p_items[x];
    prefill_tile<KV, D, G>(a, item >> kItemBits, h, item & ((1 << kItemBits) - 1), smem);
    return;
  }
  const int y = x - a.p_bound;
  if (y >= a.hdr[1]) return;
  const int item = a.d_items[y];
  const int s = item >> kItemBits, p = item & ((1 << kItemBits) - 1);
  decode_partition<KV, QT, D, G>(a.dec, s, h, p, a.qsl[s], a.dec.ctx[s], s,
                                 reinterpret_cast<float *>(smem));
}

// Decode rows split over several partitions: combine them (one group per row, head).
template <int QT, int D>
__global__ __launch_bounds__(D) void pa_mixed_decode_merge_kernel(MixedArgs a) {
  const int s = blockIdx.y;
  if (a.qsl[s + 1] - a.qsl[s] != 1) return;
  merge_partitions<QT, D>(a.dec, s, blockIdx.x, threadIdx.x, a.dec.ctx[s], a.qsl[s]);
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
static hipError_t launch_tiles(const MixedArgs &a, hipStream_t st) {
  hipLaunchKernelGGL(pa_mixed_prep_kernel, dim3(1), dim3(256), 0, st, a);
  dim3 grid(a.p_bound + a.d_bound, a.dec.num_kv_heads);
  hipLaunchKernelGGL((pa_mixed_kernel<KV, QT, D, G>), grid, dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.dec.max_parts > 1) {
    dim3 mg(a.dec.num_q_heads, a.num_seqs);
    hipLaunchKernelGGL((pa_mixed_decode_merge_kernel<QT, D>), mg, dim3(D), 0, st, a);
  }
  return hipGetLastError();
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
static hipError_t launch_g(const MixedArgs &a, int G, int num_rows, bool tiles, hipStream_t st) {
  constexpr bool kMfma = (KV == PA_F16 || KV == PA_BF16);
#define PA_CASE(g)                                                              \
  case g:                                                                       \
    if constexpr (kMfma) {                                                      \
      if (tiles) return launch_tiles<KV, QT, D, g>(a, st);                      \
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
                           hipStream_t st) {
  if (D == 64) return launch_g<KV, QT, 64>(a, G, num_rows, tiles, st);
  if (D == 128) return launch_g<KV, QT, 128>(a, G, num_rows, tiles, st);
  return hipErrorInvalidValue;
}

bool mixed_uses_tiles(int kv_dtype) { return kv_dtype == PA_F16 || kv_dtype == PA_BF16; }

hipError_t launch_mixed(const MixedArgs &a, int kv_dtype, int q_dtype, int head_dim, int group,
                        int num_rows, hipStream_t st) {
  const bool tiles = mixed_uses_tiles(kv_dtype);
  switch (kv_dtype) {
    case PA_F32: return launch_d<PA_F32, PA_F32>(a, head_dim, group, num_rows, tiles, st);
    case PA_F16: return launch_d<PA_F16, PA_F16>(a, head_dim, group, num_rows, tiles, st);
    case PA_BF16: return launch_d<PA_BF16, PA_BF16>(a, head_dim, group, num_rows, tiles, st);
    case PA_FP8_E4M3:
      return q_dtype == PA_F16
                 ? launch_d<PA_FP8_E4M3, PA_F16>(a, head_dim, group, num_rows, tiles, st)
                 : launch_d<PA_FP8_E4M3, PA_BF16>(a, head_dim, group, num_rows, tiles, st);
    case PA_I8:
      return q_dtype == PA_F16 ? launch_d<PA_I8, PA_F16>(a, head_dim, group, num_rows, tiles, st)
                               : launch_d<PA_I8, PA_BF16>(a, head_dim, group, num_rows, tiles, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
