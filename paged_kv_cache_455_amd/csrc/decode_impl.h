// Device templates of the paged decode path, shared by the decode kernel and
// the decode rows of the mixed prefill+decode kernel.
//
// What is computed ("从KV Cache到vLLM" section 1.1; 5688vip chapter 3, section
// 3.2): for every query row, each query head's dot products with all cached
// keys of its kv head, a softmax over them, and the softmax-weighted sum of the
// cached values.  Keys and values live in 16-token physical blocks found through
// the sequence's block table.
//
// Work decomposition (MI355X, wave64):
//  * one workgroup per (query row, kv head, context partition of part_blocks
//    blocks); the GQA group of G query heads shares every K/V tile load;
//  * 4 waves per workgroup; wave w takes blocks w, w+4, ... of the partition,
//    double-buffering the next tile's loads in registers while it computes;
//  * one (block, kv head) tile is 16 x head_dim contiguous elements; a
//    wave-wide load instruction reads 64 x 16 bytes (8 bytes for 1-byte codes)
//    contiguous, so lane l owns the same CB-byte column chunk of every token row
//    it touches, for K and V alike;
//  * q.k partial sums are completed with DPP adds inside each row of LPT lanes,
//    after which every lane holds the finished scores of its own tokens for all
//    G heads: the P.V update needs no further data exchange;
//  * each lane keeps its own running (max, sum, acc) over the tokens it saw; the
//    lanes' and waves' states are merged once at the end (LDS), and partitions
//    in a second kernel (or directly to the output when there is only one).
#pragma once

#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

template <int KV, int D>
struct Geom {
  static constexpr int E = dtype_bytes(KV);
  static constexpr int CB = (E == 1) ? 8 : 16;  // bytes one lane loads per instruction
  static constexpr int EPC = CB / E;            // elements per lane chunk
  static constexpr int LPT = D / EPC;           // lanes that share one token row
  static constexpr int TPI = kWave / LPT;       // token rows per wave-wide load
  static constexpr int NL = kBlock / TPI;       // loads per lane per tile
  static constexpr int TILE_BYTES = kBlock * D * E;
  static constexpr int W32 = CB / 4;            // 32-bit words per chunk
  static_assert(LPT >= 1 && LPT <= kWave && kWave % LPT == 0, "geometry");
  static_assert(NL >= 1, "geometry");
};

template <int W32>
struct Chunk {
  uint32_t w[W32];
};

template <int W32>
__device__ __forceinline__ Chunk<W32> load_chunk(const char *p) {
  Chunk<W32> c;
  if constexpr (W32 == 4) {
    u32x4 x = *reinterpret_cast<const u32x4 *>(p);
    c.w[0] = x[0]; c.w[1] = x[1]; c.w[2] = x[2]; c.w[3] = x[3];
  } else {
    u32x2 x = *reinterpret_cast<const u32x2 *>(p);
    c.w[0] = x[0]; c.w[1] = x[1];
  }
  return c;
}

// Element values of one chunk as floats.
template <int KV, int W32>
__device__ __forceinline__ void chunk_to_f32(const Chunk<W32> &c, float *f) {
  if constexpr (KV == PA_F32) {
#pragma unroll
    for (int i = 0; i < W32; ++i) f[i] = __builtin_bit_cast(float, c.w[i]);
  } else if constexpr (KV == PA_F16) {
#pragma unroll
    for (int i = 0; i < W32; ++i) { f[2 * i] = f16_lo(c.w[i]); f[2 * i + 1] = f16_hi(c.w[i]); }
  } else if constexpr (KV == PA_BF16) {
#pragma unroll
    for (int i = 0; i < W32; ++i) { f[2 * i] = bf16_lo(c.w[i]); f[2 * i + 1] = bf16_hi(c.w[i]); }
  } else if constexpr (KV == PA_FP8_E4M3) {
#pragma unroll
    for (int i = 0; i < W32; ++i) fp8x4_to_f32(c.w[i], f + 4 * i);
  } else {
#pragma unroll
    for (int i = 0; i < W32; ++i) i8x4_to_f32(c.w[i], f + 4 * i);
  }
}

// One query head's slice matching a lane chunk, in the form its dot product wants.
template <int KV, int EPC>
struct QFrag {
  // f16 / bf16 keys: packed pairs for v_dot2; otherwise floats for FMAs.
  static constexpr bool kPacked = (KV == PA_F16 || KV == PA_BF16);
  uint32_t pk[kPacked ? EPC / 2 : 1];
  float f[kPacked ? 1 : EPC];

  template <int QT>
  __device__ __forceinline__ void load(const void *q, int64_t base) {
    if constexpr (kPacked) {
      const uint32_t *p = reinterpret_cast<const uint32_t *>(
          reinterpret_cast<const char *>(q) + base * 2);
#pragma unroll
      for (int i = 0; i < EPC / 2; ++i) pk[i] = p[i];
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) f[i] = load_q<QT>(q, base + i);
    }
  }

  // Partial dot product of this slice with the key chunk.
  template <int W32>
  __device__ __forceinline__ float dot(const Chunk<W32> &k, const float *kf) const {
    float acc = 0.f;
    if constexpr (KV == PA_F16) {
#pragma unroll
      for (int i = 0; i < W32; ++i)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, k.w[i]),
                                     __builtin_bit_cast(h2_t, pk[i]), acc, false);
    } else if constexpr (KV == PA_BF16) {
#pragma unroll
      for (int i = 0; i < W32; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2_t, k.w[i]),
                                              __builtin_bit_cast(bf2_t, pk[i]), acc, false);
    } else {
#pragma unroll
      for (int i = 0; i < EPC; ++i) acc = __builtin_fmaf(f[i], kf[i], acc);
    }
    return acc;
  }
};

template <int KV, int QT, int D, int G>
struct DecodeState {
  using Gm = Geom<KV, D>;
  QFrag<KV, Gm::EPC> q[G];
  float m[G], l[G];
  float acc[G][Gm::EPC];
};

// Online-softmax update of one lane with one (block, kv head) tile.
template <int KV, int QT, int D, int G, bool MASK>
__device__ __forceinline__ void tile_update(DecodeState<KV, QT, D, G> &st,
                                            const Chunk<Geom<KV, D>::W32> *kc,
                                            const Chunk<Geom<KV, D>::W32> *vc, float qk_scale,
                                            float v_scale, int valid_rows, int tg) {
  using Gm = Geom<KV, D>;
  constexpr int NL = Gm::NL, EPC = Gm::EPC, W32 = Gm::W32;
  constexpr bool kNeedKf = !(KV == PA_F16 || KV == PA_BF16);
  float s[NL][G];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    float kf[kNeedKf ? EPC : 1];
    if constexpr (kNeedKf) chunk_to_f32<KV, W32>(kc[i], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) s[i][g] = st.q[g].dot(kc[i], kf);
  }
#pragma unroll
  for (int i = 0; i < NL; ++i)
#pragma unroll
    for (int g = 0; g < G; ++g) s[i][g] = group_sum<Gm::LPT>(s[i][g]) * qk_scale;

  bool valid[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i) valid[i] = !MASK || (i * Gm::TPI + tg) < valid_rows;
  if constexpr (MASK) {
#pragma unroll
    for (int i = 0; i < NL; ++i)
#pragma unroll
      for (int g = 0; g < G; ++g) s[i][g] = valid[i] ? s[i][g] : kNegBig;
  }

  float vf[NL][EPC];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    Chunk<W32> c = vc[i];
    if constexpr (MASK) {
      // rows past the context may hold anything (NaN included): zero their bits
#pragma unroll
      for (int w = 0; w < W32; ++w) c.w[w] = valid[i] ? c.w[w] : 0u;
    }
    chunk_to_f32<KV, W32>(c, vf[i]);
  }

#pragma unroll
  for (int g = 0; g < G; ++g) {
    float mt = s[0][g];
#pragma unroll
    for (int i = 1; i < NL; ++i) mt = fmaxf(mt, s[i][g]);
    const float mn = fmaxf(st.m[g], mt);
    const float alpha = fast_exp2(st.m[g] - mn);
    st.m[g] = mn;
    float p[NL];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      p[i] = fast_exp2(s[i][g] - mn);
      if constexpr (MASK) p[i] = valid[i] ? p[i] : 0.f;
      psum += p[i];
    }
    st.l[g] = st.l[g] * alpha + psum;
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float a = st.acc[g][e] * alpha;
#pragma unroll
      for (int i = 0; i < NL; ++i) a = __builtin_fmaf(p[i] * v_scale, vf[i][e], a);
      st.acc[g][e] = a;
    }
  }
}

// Combine two online-softmax states (m1, l1, a1) <- (m1, l1, a1) (+) (m2, l2, a2).
__device__ __forceinline__ void merge_weights(float m1, float m2, float &w1, float &w2, float &mn) {
  mn = fmaxf(m1, m2);
  w1 = fast_exp2(m1 - mn);
  w2 = fast_exp2(m2 - mn);
}

constexpr int kDecodeWaves = 4;

// One workgroup: query row q_row of sequence s (block-table row), kv head h,
// context partition p, attending to the first n cached tokens.  Partial states
// go to workspace row ws_row.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void decode_partition(const DecodeArgs &a, int s, int h, int p,
                                                 int q_row, int n, int ws_row) {
  using Gm = Geom<KV, D>;
  constexpr int NL = Gm::NL, EPC = Gm::EPC, W32 = Gm::W32, LPT = Gm::LPT;
  constexpr int NW = kDecodeWaves;
  const int hq0 = h * G;
  const int64_t out_base = ((int64_t)q_row * a.num_q_heads + hq0) * D;
  if (n <= 0) {  // undefined input; keep the output finite and defined
    if (p == 0)
      for (int i = threadIdx.x; i < G * D; i += blockDim.x) store_out<QT>(a.out, out_base + i, 0.f);
    return;
  }
  const int nblk = (n + kBlock - 1) / kBlock;
  const int jbeg = p * a.part_blocks;
  if (jbeg >= nblk) return;
  const int jend = min(jbeg + a.part_blocks, nblk);
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int cidx = lane % LPT;  // column chunk
  const int tg = lane / LPT;    // token group

  DecodeState<KV, QT, D, G> st;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st.q[g].template load<QT>(a.q, out_base + (int64_t)g * D + cidx * EPC);
    st.m[g] = kNegBig;
    st.l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) st.acc[g][e] = 0.f;
  }

  const int32_t *bt = a.bt + (int64_t)s * a.max_blocks_per_seq;
  const char *kbase = reinterpret_cast<const char *>(a.k);
  const char *vbase = reinterpret_cast<const char *>(a.v);
  const int lane_off = lane * Gm::CB;
  const int last_blk = nblk - 1;
  const int tail_rows = n - last_blk * kBlock;  // 1..16 rows valid in the last block
  const bool quant = (KV == PA_FP8_E4M3 || KV == PA_I8);

  Chunk<W32> kA[NL], vA[NL], kB[NL], vB[NL];
  float ksA = 1.f, vsA = 1.f, ksB = 1.f, vsB = 1.f;

  auto load_tile = [&](int j, Chunk<W32> *kc, Chunk<W32> *vc, float &ks, float &vs) {
    const int64_t tile = (int64_t)bt[j] * a.num_kv_heads + h;
    const char *kp = kbase + tile * Gm::TILE_BYTES + lane_off;
    const char *vp = vbase + tile * Gm::TILE_BYTES + lane_off;
#pragma unroll
    for (int i = 0; i < NL; ++i) kc[i] = load_chunk<W32>(kp + i * kWave * Gm::CB);
#pragma unroll
    for (int i = 0; i < NL; ++i) vc[i] = load_chunk<W32>(vp + i * kWave * Gm::CB);
    if (quant) {
      ks = a.k_scale[tile];
      vs = a.v_scale[tile];
    }
  };
  auto compute = [&](int j, const Chunk<W32> *kc, const Chunk<W32> *vc, float ks, float vs) {
    const float qs = a.qk_scale * ks;
    if (j == last_blk && tail_rows < kBlock)
      tile_update<KV, QT, D, G, true>(st, kc, vc, qs, vs, tail_rows, tg);
    else
      tile_update<KV, QT, D, G, false>(st, kc, vc, qs, vs, kBlock, tg);
  };

  int j = jbeg + wave;
  if (j < jend) {
    load_tile(j, kA, vA, ksA, vsA);
    for (;;) {
      int jn = j + NW;
      if (jn < jend) load_tile(jn, kB, vB, ksB, vsB);
      compute(j, kA, vA, ksA, vsA);
      j = jn;
      if (j >= jend) break;
      jn = j + NW;
      if (jn < jend) load_tile(jn, kA, vA, ksA, vsA);
      compute(j, kB, vB, ksB, vsB);
      j = jn;
      if (j >= jend) break;
    }
  }

  // ---- merge the token groups of this wave (lanes that differ in tg) ----
#pragma unroll
  for (int mask = LPT; mask < kWave; mask <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(st.m[g], mask, kWave);
      const float lo = __shfl_xor(st.l[g], mask, kWave);
      float w1, w2, mn;
      merge_weights(st.m[g], mo, w1, w2, mn);
      st.m[g] = mn;
      st.l[g] = st.l[g] * w1 + lo * w2;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float ao = __shfl_xor(st.acc[g][e], mask, kWave);
        st.acc[g][e] = st.acc[g][e] * w1 + ao * w2;
      }
    }
  }

  // ---- merge the waves through LDS ----
  __shared__ float sm_acc[NW][G][D];
  __shared__ float sm_m[NW][G];
  __shared__ float sm_l[NW][G];
  if (tg == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) sm_acc[wave][g][cidx * EPC + e] = st.acc[g][e];
      if (cidx == 0) {
        sm_m[wave][g] = st.m[g];
        sm_l[wave][g] = st.l[g];
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int g = i / D, d = i % D;
    float M = sm_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = fast_exp2(sm_m[w][g] - M);
      L += wt * sm_l[w][g];
      A += wt * sm_acc[w][g][d];
    }
    if (nparts == 1) {
      store_out<QT>(a.out, out_base + i, A / L);
    } else {
      const int64_t r = ((int64_t)ws_row * a.num_q_heads + hq0 + g) * a.max_parts + p;
      a.ws_acc[r * D + d] = A;
      if (d == 0) {
        a.ws_m[r] = M;
        a.ws_l[r] = L;
      }
    }
  }
}

// Combine the partitions of workspace row r for query head hq, one thread per
// output element d (second pass).  With per-partition (m_p, l_p, acc_p):
//   M = max_p m_p,  L = sum_p 2^(m_p - M) l_p,  out = sum_p 2^(m_p - M) acc_p / L.
// Rows whose context fits in one partition were finished by the first pass.
template <int QT, int D>
__device__ __forceinline__ void merge_partitions(const DecodeArgs &a, int r, int hq, int d, int n,
                                                 int q_row = -1) {
  if (n <= 0) return;
  const int nblk = (n + kBlock - 1) / kBlock;
  const int nparts = (nblk + a.part_blocks - 1) / a.part_blocks;
  if (nparts <= 1) return;
  if (q_row < 0) q_row = r;
  const int64_t r0 = ((int64_t)r * a.num_q_heads + hq) * a.max_parts;
  float M = kNegBig;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_m[r0 + p]);
  float L = 0.f, A = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float wt = fast_exp2(a.ws_m[r0 + p] - M);
    L += wt * a.ws_l[r0 + p];
    A += wt * a.ws_acc[(r0 + p) * D + d];
  }
  store_out<QT>(a.out, ((int64_t)q_row * a.num_q_heads + hq) * D + d, A / L);
}

}  // namespace pa
