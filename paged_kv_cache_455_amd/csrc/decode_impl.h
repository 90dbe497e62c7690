// Device templates of the paged decode path, shared by the decode kernel and
// the decode rows of the mixed prefill+decode kernel.
//
// What is computed ("从KV Cache到vLLM" section 1.1; 5688vip chapter 3, section
// 3.2): for every query row, each query head's dot products with all cached
// keys of its kv head, a softmax over them, and the softmax-weighted sum of the
// cached values.  Keys and values live in 16-token physical blocks found through
// the sequence's block table.
//
// Work decomposition (MI355X, wave64).  Two forms share the per-tile code:
//  * the balanced split (pa_decode, the mixed step's one-token rows; see
//    stream_range / stream_run below): every (sequence, kv head, 16-row tile) of
//    the batch forms one list and each wave of a grid sized to the resident
//    capacity streams an equal share of it, emitting a finished output for a
//    segment it owns alone and a partial (m, l, acc) piece otherwise, merged by a
//    second kernel;
//  * the partitioned form (decode_partition; the mixed step's rows for fp32 KV):
//    one workgroup per (query row, kv head, context partition), 4 waves taking
//    blocks w, w+4, ... and merging through LDS.
// In both, the GQA group of G query heads shares every K/V tile load; one
// (block, kv head) tile is 16 x head_dim contiguous elements, and a wave-wide
// load instruction reads 64 x 16 bytes (8 bytes for 1-byte codes) contiguous, so
// lane l owns the same CB-byte column chunk of every token row it touches, for K
// and V alike; q.k partial sums are completed with DPP adds inside each row of
// LPT lanes, after which the lanes hold finished scores for the P.V update; each
// lane keeps its own running (max, sum, acc), merged across lanes at the end.
// Where that vector work per tile, not the loads, would set the pace -- 1-byte KV
// at GQA groups 2-8, 16-bit KV at groups 4 and 8, both widths at head_dim 64 and
// groups 2-8 (MxGeom) -- the balanced split runs both products of a tile on MFMA
// instead (MxPath below).
#pragma once

#include <type_traits>

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

// K/V tile loads.  A tile that one call reads once is loaded with the nontemporal
// hint (NT), which streams it past the caches: measured on MI355X, a gather of 8 KiB
// tiles runs at about 6.9 TB/s with it against 5.8-6.0 TB/s without.  Tiles that
// several sequences share (prefix sharing) are read with ordinary loads instead, so
// that their repeated reads can hit in L2 and the Infinity Cache.
template <class T, bool NT>
__device__ __forceinline__ T load_tile_part(const char *p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const T *>(p));
  else
    return *reinterpret_cast<const T *>(p);
}

template <int W32, bool NT = true>
__device__ __forceinline__ Chunk<W32> load_chunk(const char *p) {
  Chunk<W32> c;
  if constexpr (W32 == 4) {
    const u32x4 x = load_tile_part<u32x4, NT>(p);
    c.w[0] = x[0]; c.w[1] = x[1]; c.w[2] = x[2]; c.w[3] = x[3];
  } else {
    const u32x2 x = load_tile_part<u32x2, NT>(p);
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

// ---- fast path for 16-lane token rows (LPT == 16, 4 loads per tile) and G >= 4 ------
// After the partial dot products every lane of a row holds NV = 4*G partial sums;
// a reduce-scatter leaves each lane NV/16 finished scores, so each score's exp is
// computed once.  The probabilities and rescale factors then go back to every lane
// of the row by DPP row broadcasts for the P.V update.
template <int KV, int D, int G>
struct FastGeom {
  static constexpr bool kOn = Geom<KV, D>::LPT == 16 && Geom<KV, D>::NL == 4 && (G == 4 || G == 8);
  static constexpr int NV = 4 * G;    // partial values per lane before the reduce-scatter
  static constexpr int NVL = NV / 16; // finished scores per lane after it
};

template <int KV, int D, int G>
struct FastState {
  static constexpr int NVL = FastGeom<KV, D, G>::NVL;
  float m[NVL], l[NVL];  // running max / sum for this lane's heads, shared by its row
};

// Lane c of row r owns, after the reduce-scatter, value indices v = c*NVL + j, i.e.
// load slot i = c/4 (token 4*(c/4) + r) and heads g = v % G.
template <int KV, int QT, int D, int G, bool MASK>
__device__ __forceinline__ void tile_update_fast(DecodeState<KV, QT, D, G> &st,
                                                 FastState<KV, D, G> &fs,
                                                 const Chunk<Geom<KV, D>::W32> *kc,
                                                 const Chunk<Geom<KV, D>::W32> *vc,
                                                 float qk_scale, float v_scale, int valid_rows,
                                                 int r, int c) {
  using Gm = Geom<KV, D>;
  using Fg = FastGeom<KV, D, G>;
  constexpr int NL = Gm::NL, EPC = Gm::EPC, W32 = Gm::W32, NV = Fg::NV, NVL = Fg::NVL;
  constexpr bool kNeedKf = !(KV == PA_F16 || KV == PA_BF16);
  constexpr bool kQuant = (KV == PA_FP8_E4M3 || KV == PA_I8);
  float part[NV];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    float kf[kNeedKf ? EPC : 1];
    if constexpr (kNeedKf) chunk_to_f32<KV, W32>(kc[i], kf);
#pragma unroll
    for (int g = 0; g < G; ++g) part[i * G + g] = st.q[g].dot(kc[i], kf);
  }
  row_reduce_scatter<NV>(part, c);

  const bool valid = !MASK || (4 * (c >> 2) + r) < valid_rows;
  float p[NVL];
  bool changed = false;
#pragma unroll
  for (int j = 0; j < NVL; ++j) {
    float s = part[j] * qk_scale;
    if constexpr (MASK) s = valid ? s : kNegBig;
    float mt = fmaxf(s, dpp_f<kDppRor4>(s));
    mt = fmaxf(mt, dpp_f<kDppRor8>(mt));
    const float mn = fmaxf(fs.m[j], mt);
    changed |= mn > fs.m[j];
    const float alpha = fast_exp2(fs.m[j] - mn);
    float pj = fast_exp2(s - mn);
    if constexpr (MASK) pj = valid ? pj : 0.f;
    fs.l[j] = fs.l[j] * alpha + pj;
    fs.m[j] = mn;
    part[NVL + j] = alpha;       // park alpha next to the score slots
    p[j] = kQuant ? pj * v_scale : pj;
  }
  if (__any(changed)) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float a;
      // alpha of head g lives in lane g / NVL (token slot 0), slot g % NVL
#define PA_BC(n) case n: a = row_bcast<n>(part[NVL + g % NVL]); break;
      switch (g / NVL) { PA_BC(0) PA_BC(1) PA_BC(2) PA_BC(3) PA_BC(4) PA_BC(5) PA_BC(6) PA_BC(7) default: a = 1.f; }
#undef PA_BC
#pragma unroll
      for (int e = 0; e < EPC; ++e) st.acc[g][e] *= a;
    }
  }
  float P[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
#define PA_BC(n) case n: P[v] = row_bcast<n>(p[v % NVL]); break;
    switch (v / NVL) {
      PA_BC(0) PA_BC(1) PA_BC(2) PA_BC(3) PA_BC(4) PA_BC(5) PA_BC(6) PA_BC(7)
      PA_BC(8) PA_BC(9) PA_BC(10) PA_BC(11) PA_BC(12) PA_BC(13) PA_BC(14) PA_BC(15)
    }
#undef PA_BC
  }

  const int tg = r;
  float vf[NL][EPC];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    Chunk<W32> cv = vc[i];
    if constexpr (MASK) {
      const bool ok = (i * Gm::TPI + tg) < valid_rows;
#pragma unroll
      for (int w = 0; w < W32; ++w) cv.w[w] = ok ? cv.w[w] : 0u;
    }
    chunk_to_f32<KV, W32>(cv, vf[i]);
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float a = st.acc[g][e];
#pragma unroll
      for (int i = 0; i < NL; ++i) a = __builtin_fmaf(P[i * G + g], vf[i][e], a);
      st.acc[g][e] = a;
    }
}

// Turn the fast per-lane state into the generic one (m[G], l[G] shared by a row).
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void fast_to_generic(DecodeState<KV, QT, D, G> &st,
                                                FastState<KV, D, G> &fs) {
  constexpr int NVL = FastGeom<KV, D, G>::NVL;
#pragma unroll
  for (int j = 0; j < NVL; ++j) {  // sum the four token slots' partial l (same max)
    fs.l[j] += dpp_f<kDppRor4>(fs.l[j]);
    fs.l[j] += dpp_f<kDppRor8>(fs.l[j]);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#define PA_BC(n) case n: st.m[g] = row_bcast<n>(fs.m[g % NVL]); st.l[g] = row_bcast<n>(fs.l[g % NVL]); break;
    switch (g / NVL) { PA_BC(0) PA_BC(1) PA_BC(2) PA_BC(3) PA_BC(4) PA_BC(5) PA_BC(6) PA_BC(7) }
#undef PA_BC
  }
}

// Combine two online-softmax states (m1, l1, a1) <- (m1, l1, a1) (+) (m2, l2, a2).
__device__ __forceinline__ void merge_weights(float m1, float m2, float &w1, float &w2, float &mn) {
  mn = fmaxf(m1, m2);
  w1 = fast_exp2(m1 - mn);
  w2 = fast_exp2(m2 - mn);
}

// One step of the token-group merge: combine with the lanes MASK apart, then the
// next higher lane bit, up to 32 (cross-lane moves without LDS).
template <int MASK, int KV, int QT, int D, int G>
__device__ __forceinline__ void merge_token_step(DecodeState<KV, QT, D, G> &st) {
  if constexpr (MASK < kWave) {
    constexpr int EPC = Geom<KV, D>::EPC;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = xor_lanes<MASK>(st.m[g]);
      const float lo = xor_lanes<MASK>(st.l[g]);
      float w1, w2, mn;
      merge_weights(st.m[g], mo, w1, w2, mn);
      st.m[g] = mn;
      st.l[g] = st.l[g] * w1 + lo * w2;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float ao = xor_lanes<MASK>(st.acc[g][e]);
        st.acc[g][e] = st.acc[g][e] * w1 + ao * w2;
      }
    }
    merge_token_step<MASK * 2>(st);
  }
}

// Merge the token groups of one wave (lanes that differ above the LPT lanes of a
// row) so that every lane ends with the wave's (m, l, acc) for its column chunk.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void merge_token_groups(DecodeState<KV, QT, D, G> &st) {
  constexpr int LPT = Geom<KV, D>::LPT;
  merge_token_step<LPT>(st);
}

constexpr int kDecodeWaves = 4;

// LDS floats decode_partition needs for its cross-wave merge.
template <int D, int G>
constexpr int decode_partition_smem_floats() {
  return kDecodeWaves * G * D + 2 * kDecodeWaves * G;
}

// One workgroup: query row q_row of sequence s (block-table row), kv head h,
// context partition p, attending to the first n cached tokens.  Partial states
// go to workspace row ws_row.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void decode_partition(const DecodeArgs &a, int s, int h, int p,
                                                 int q_row, int n, int ws_row, float *smem) {
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
    const int64_t tile = tile_index(bt[j >> a.bs_shift], a.num_kv_heads, h, j, a.bs_shift);
    const char *kp = kbase + tile * Gm::TILE_BYTES + lane_off;
    const char *vp = vbase + tile * Gm::TILE_BYTES + lane_off;
#pragma unroll
    for (int i = 0; i < NL; ++i) kc[i] = load_chunk<W32>(kp + i * kWave * Gm::CB);
#pragma unroll
    for (int i = 0; i < NL; ++i) vc[i] = load_chunk<W32>(vp + i * kWave * Gm::CB);
    if (quant) {
      ks = a.k_scale[tile >> a.bs_shift];
      vs = a.v_scale[tile >> a.bs_shift];
    }
  };
  constexpr bool kFast = FastGeom<KV, D, G>::kOn;
  FastState<KV, D, G> fs;
#pragma unroll
  for (int j = 0; j < FastGeom<KV, D, G>::NVL; ++j) {
    fs.m[j] = kNegBig;
    fs.l[j] = 0.f;
  }
  auto compute = [&](int j, const Chunk<W32> *kc, const Chunk<W32> *vc, float ks, float vs) {
    const float qs = quant ? a.qk_scale * ks : a.qk_scale;
    if constexpr (kFast) {
      if (j == last_blk && tail_rows < kBlock)
        tile_update_fast<KV, QT, D, G, true>(st, fs, kc, vc, qs, vs, tail_rows, tg, cidx);
      else
        tile_update_fast<KV, QT, D, G, false>(st, fs, kc, vc, qs, vs, kBlock, tg, cidx);
    } else {
      if (j == last_blk && tail_rows < kBlock)
        tile_update<KV, QT, D, G, true>(st, kc, vc, qs, vs, tail_rows, tg);
      else
        tile_update<KV, QT, D, G, false>(st, kc, vc, qs, vs, kBlock, tg);
    }
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

  if constexpr (kFast) fast_to_generic(st, fs);

  merge_token_groups(st);

  // ---- merge the waves through LDS (smem: NW*G*D + 2*NW*G floats) ----
  float(*sm_acc)[G][D] = reinterpret_cast<float(*)[G][D]>(smem);
  float(*sm_m)[G] = reinterpret_cast<float(*)[G]>(smem + NW * G * D);
  float(*sm_l)[G] = reinterpret_cast<float(*)[G]>(smem + NW * G * D + NW * G);
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

// ---- balanced split ("stream" decode) ------------------------------------------------
// All (sequence, kv head, block) tiles of the batch form one list, ordered by
// sequence, then kv head, then block: sequence s owns blocks [cum[s], cum[s+1]) of
// the concatenated tables and its kv head h the tiles
//   [Hkv*cum[s] + h*nblk_s, Hkv*cum[s] + (h+1)*nblk_s).
// Wave w of the grid takes the tiles [w*tpw, (w+1)*tpw), tpw = max(min_tpw,
// ceil(T / waves)): every wave streams the same number of K/V bytes whatever the
// context lengths (with two workgroups per CU, the first round's waves a few
// percent more and the second round's as many fewer; see stream_range).  A wave
// emits one result per (sequence, kv head) segment it touches: the final output
// when it owns the whole segment, else a partial (m, l, acc) for "piece"
// w - first_wave(segment), combined by the merge kernel.

// Cross-lane integer steps of the split, all DPP moves between registers (a lane
// shuffle goes through the LDS crossbar: six dependent ones cost about 0.3 us).
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_i(int x) {  // lanes with no source (or masked rows) read 0
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111;     // + n - 1: lane i <- lane i - n within 16 (none below)
constexpr int kDppRowBcast15 = 0x142;  // rows 1, 2, 3 <- lane 15 of the row before
constexpr int kDppRowBcast31 = 0x143;  // rows 2, 3 <- lane 31

// The maximum over the wave (uniform): each 16-lane row folded in registers, then
// the four row maxima read by readlane.
__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<kDppXor1>(x));
  x = max(x, dpp_i<kDppXor2>(x));
  x = max(x, dpp_i<kDppHalfMirror>(x));  // quads agree: pairs quad 0 with quad 1
  x = max(x, dpp_i<kDppMirror>(x));      // halves agree: pairs the two halves
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}
// Inclusive prefix sum over the lanes: a scan of each row by shifts of 1, 2, 4 and 8
// (zeros shifted in), then each row's total carried into the rows after it.
__device__ __forceinline__ int wave_incl_scan_i(int x, int lane) {
  (void)lane;
  x += dpp_i<kDppRowShr1>(x);
  x += dpp_i<kDppRowShr1 + 1>(x);
  x += dpp_i<kDppRowShr1 + 3>(x);
  x += dpp_i<kDppRowShr1 + 7>(x);
  x += dpp_i<kDppRowBcast15, 0xa>(x);  // rows 1 and 3 take the totals of rows 0 and 2
  x += dpp_i<kDppRowBcast31, 0xc>(x);  // rows 2 and 3 take the total of rows 0..1
  return x;
}

// Decode rows of a mixed step: with a.qsl set, sequence s's query row is qsl[s] and
// only sequences with one new token (q_len == 1) take part; without it sequence s
// is row s.
__device__ __forceinline__ int decode_len(const DecodeArgs &a, int s) {
  if (a.qsl != nullptr && a.qsl[s + 1] - a.qsl[s] != 1) return 0;
  return a.ctx[s];
}
__device__ __forceinline__ int64_t decode_row(const DecodeArgs &a, int s) {
  return a.qsl != nullptr ? a.qsl[s] : s;
}
// The same for a wave-uniform s, by a scalar load: its wait counts scalar loads only,
// so it does not drain the K/V loads in flight (a vector load behind the test of
// qsl makes the compiler wait for every vector load on both paths).
__device__ __forceinline__ int64_t decode_row_uniform(const DecodeArgs &a, int s) {
  if (a.qsl == nullptr) return s;
  using cint = const __attribute__((address_space(4))) int;
  return *(cint *)(a.qsl + __builtin_amdgcn_readfirstlane(s));
}

// Write this wave's state for (s, kv head h): normalised output when single,
// else the partial for `piece`.  Lanes of token group 0 hold every column chunk.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void emit_segment(const DecodeArgs &a, DecodeState<KV, QT, D, G> &st,
                                             int s, int h, bool single, int piece, int lane) {
  const int64_t row = decode_row(a, s);
  constexpr int EPC = Geom<KV, D>::EPC, LPT = Geom<KV, D>::LPT;
  merge_token_groups(st);
  if (lane >= LPT) return;
  const int c = lane;
  if (single) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = 1.f / st.l[g];
      const int64_t o = (row * a.num_q_heads + h * G + g) * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) store_out<QT>(a.out, o + e, st.acc[g][e] * inv);
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t r = ((int64_t)s * a.num_q_heads + h * G + g) * a.max_parts + piece;
      float *dst = a.ws_acc + r * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = st.acc[g][e];
      if (c == 0) {
        a.ws_m[r] = st.m[g];
        a.ws_l[r] = st.l[g];
      }
    }
  }
}

// emit_segment for waves of four token groups (rows of 16 lanes) and a group of
// 4 or 8 heads, by reduce-scatter instead of the all-reduce above: step 1 merges
// rows r and r^1, the even row keeping heads [0, G/2) and the odd row heads
// [G/2, G); step 2 merges the halves, the lower keeping the first half of what is
// left.  Each lane ends with G/4 heads (head q + G/4*(r>>1) + G/2*(r&1) in slot q)
// for its column chunk, and every lane stores: a quarter of the cross-lane moves
// and merge arithmetic of the all-reduce, which kept four copies of everything.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void emit_segment_rs(const DecodeArgs &a, DecodeState<KV, QT, D, G> &st,
                                                int s, int h, bool single, int piece, int lane) {
  constexpr int EPC = Geom<KV, D>::EPC, G2 = G / 2, G4 = G / 4;
  static_assert(Geom<KV, D>::LPT == 16 && G % 4 == 0, "four token rows, G a multiple of 4");
  // merge state (mx, lx, ax) with (my, ly, ay) into x
  auto merge = [](float &mx, float my, float &lx, float ly, float *ax, const float *ay) {
    const float mn = fmaxf(mx, my);
    const float wx = fast_exp2(mx - mn), wy = fast_exp2(my - mn);
    mx = mn;
    lx = lx * wx + ly * wy;
#pragma unroll
    for (int e = 0; e < EPC; ++e) ax[e] = ax[e] * wx + ay[e] * wy;
  };
#pragma unroll
  for (int p = 0; p < G2; ++p) {
    swap_rows<16>(st.m[p], st.m[p + G2]);
    swap_rows<16>(st.l[p], st.l[p + G2]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) swap_rows<16>(st.acc[p][e], st.acc[p + G2][e]);
    merge(st.m[p], st.m[p + G2], st.l[p], st.l[p + G2], st.acc[p], st.acc[p + G2]);
  }
#pragma unroll
  for (int q = 0; q < G4; ++q) {
    swap_rows<32>(st.m[q], st.m[q + G4]);
    swap_rows<32>(st.l[q], st.l[q + G4]);
#pragma unroll
    for (int e = 0; e < EPC; ++e) swap_rows<32>(st.acc[q][e], st.acc[q + G4][e]);
    merge(st.m[q], st.m[q + G4], st.l[q], st.l[q + G4], st.acc[q], st.acc[q + G4]);
  }
  const int r = lane >> 4, c = lane & 15;
  const int g0 = G4 * (r >> 1) + G2 * (r & 1);
#pragma unroll
  for (int q = 0; q < G4; ++q) {
    const int g = g0 + q;
    if (single) {
      const float inv = 1.f / st.l[q];
      const int64_t o = (decode_row_uniform(a, s) * a.num_q_heads + h * G + g) * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) store_out<QT>(a.out, o + e, st.acc[q][e] * inv);
    } else {
      const int64_t w = ((int64_t)s * a.num_q_heads + h * G + g) * a.max_parts + piece;
      float *dst = a.ws_acc + w * D + c * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = st.acc[q][e];
      if (c == 0) {
        a.ws_m[w] = st.m[q];
        a.ws_l[w] = st.l[q];
      }
    }
  }
}

// ---- balanced split: the wave's range of tiles ---------------------------------------
struct StreamSeg {
  int s, h;   // sequence, kv head
  int nblk;   // blocks of the sequence
  int cum;    // cost units of the sequences before it
  int tail;   // valid rows of its last block
};

// Context lengths of the sequences [s0, s0 + 64), one per lane (0 past the batch),
// read back by readlane: walking from segment to segment costs no memory round trip
// until the wave leaves the window.
struct SeqWindow {
  int s0, ctx_l;
  __device__ __forceinline__ void load(const DecodeArgs &a, int first, int lane) {
    s0 = first;
    ctx_l = first + lane < a.num_seqs ? decode_len(a, first + lane) : 0;
  }
  __device__ __forceinline__ int ctx(const DecodeArgs &a, int s, int lane) {
    if (s - s0 >= kWave) load(a, s, lane);
    return __builtin_amdgcn_readlane(ctx_l, s - s0);
  }
};

// The split of the cost units over the waves: waves [0, H) take t1 units each and
// waves [H, W) t2 (t1 = t2, H = W without a skew).
struct SplitGeom {
  int t1, t2, H;
  __device__ __forceinline__ int start(int w) const {
    return w < H ? w * t1 : H * t1 + (w - H) * t2;
  }
  __device__ __forceinline__ int wave_of(int u) const {  // the wave owning unit u
    const int b = H * t1;
    return u < b ? u / t1 : H + (u - b) / t2;
  }
};

struct StreamRange {
  SplitGeom sp;   // cost units per wave
  int n;          // tiles of the wave
  int j;          // block of the wave's first tile inside its segment
  StreamSeg seg;  // the first tile's segment
  SeqWindow win;  // context lengths of the 64 sequences from the window holding seg.s
};

// Move sg to the first segment of the next sequence that has blocks (one exists).
__device__ __forceinline__ void next_sequence(const DecodeArgs &a, SeqWindow &win, StreamSeg &sg,
                                              int lane) {
  sg.h = 0;
  sg.cum += a.num_kv_heads * (sg.nblk + a.seg_cost);
  int n, nb;
  do {  // bounded by the batch: callers only step to a sequence that exists
    ++sg.s;
    n = win.ctx(a, sg.s, lane);
    nb = n > 0 ? (n + kBlock - 1) / kBlock : 0;
  } while (nb == 0 && sg.s < a.num_seqs - 1);
  sg.nblk = max(nb, 1);
  sg.tail = n - (sg.nblk - 1) * kBlock;
}

// Cost of the work: each (sequence, kv head) segment counts seg_cost units for its
// start (the result it emits, the switch of q) plus one per tile, and waves take
// equal ranges of cost units.  Segment (s, h) covers units
// [cum_s + h*L_s, cum_s + (h+1)*L_s), L_s = nblk_s + seg_cost, its tile j sitting
// at cum_s + h*L_s + seg_cost + j; a wave owns the tiles whose units fall in its
// range.
//
// stream_range counts the batch's cost, records the units per wave (both rounds)
// and every sequence's first cost unit (wave 0 does), finds wave w's first tile
// and counts its tiles.  False
// when the wave has no tiles.  Everything it returns is wave-uniform and taken
// from lanes by readlane, so the compiler keeps the tile cursor in scalar
// registers: block-table entries, context lengths and scales are then scalar loads,
// which do not wait behind the vector K/V loads in flight.
__device__ __forceinline__ bool stream_range(const DecodeArgs &a, int w, int lane, StreamRange &r) {
  const int Hkv = a.num_kv_heads, S = a.num_seqs, c = a.seg_cost;
  auto seq_cost = [&](int nb) { return nb > 0 ? Hkv * (nb + c) : 0; };
  auto blocks = [](int n) { return n > 0 ? (n + kBlock - 1) / kBlock : 0; };
  // The lengths of the first kHeld windows of 64 sequences are read together (one
  // round trip, indices clamped into the batch) and kept, with their scan, for the
  // locate pass; longer batches read the rest window by window.
  constexpr int kHeld = 8;
  int held_n[kHeld], held_incl[kHeld];
#pragma unroll
  for (int i = 0; i < kHeld; ++i) held_n[i] = decode_len(a, min(i * kWave + lane, S - 1));
  int TC = 0, mxnb = 0;
  auto scan_window = [&](int c0, int n) {
    const int sq = c0 + lane;
    const int nb = sq < S ? blocks(n) : 0;
    mxnb = max(mxnb, nb);
    const int incl = TC + wave_incl_scan_i(seq_cost(nb), lane);
    if (w == 0 && sq < S) a.hdr[1 + sq] = incl - seq_cost(nb);
    TC = __builtin_amdgcn_readlane(incl, kWave - 1);
    return incl;
  };
#pragma unroll
  for (int i = 0; i < kHeld; ++i)
    if (i * kWave < S) held_incl[i] = scan_window(i * kWave, held_n[i]);
  for (int c0 = kHeld * kWave; c0 < S; c0 += kWave)
    scan_window(c0, c0 + lane < S ? decode_len(a, c0 + lane) : 0);
  const int base = max(a.min_tpw, (TC + a.num_waves - 1) / a.num_waves);
  // A segment of nblk tiles meets at most floor((nblk - 1) / t) + 2 waves of t units
  // or more; so with t >= ceil(max nblk / (max_parts - 1)) its pieces fit the workspace's
  // max_parts rows whatever the lengths (max_parts >= 2 by construction), also
  // when the host's length bound is low or a captured step is replayed on
  // longer contexts.
  mxnb = wave_max_i(mxnb);
  const int bound = (mxnb + a.max_parts - 2) / (a.max_parts - 1);
  // With two workgroups per CU the second wave of each SIMD issues behind the first
  // and streams slower, so the first round (waves [0, W/2): the grid's first
  // workgroups) takes d units more and the second d fewer; W/2 (t1 + t2) = W base
  // still covers TC (W is even), and t2 >= bound keeps the pieces bound.
  const int d = (base * a.skew) >> 8;
  r.sp.t1 = max(base + d, bound);
  r.sp.t2 = max(base - d, bound);
  r.sp.H = a.skew > 0 ? a.num_waves / 2 : a.num_waves;
  if (w == 0 && lane == 0) {
    a.hdr[0] = r.sp.t1;
    a.hdr[1 + S] = r.sp.t2;
  }
  const int t = r.sp.start(w);
  const int tend = min(t + (w < r.sp.H ? r.sp.t1 : r.sp.t2), TC);
  if (t >= tend) return false;

  // locate the sequence holding unit t (a hit always comes: t < TC)
  int s = 0, cum_s = 0, nblk = 1, ns = 1;
  bool found = false;
  r.win.s0 = 0;
  r.win.ctx_l = held_n[0];
  auto try_window = [&](int c0, int n, int incl) {
    const int sq = c0 + lane;
    const int nb = sq < S ? blocks(n) : 0;
    const int excl = incl - seq_cost(nb);
    const unsigned long long hit = __ballot(sq < S && nb > 0 && excl <= t && t < incl);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      s = c0 + l;
      cum_s = __builtin_amdgcn_readlane(excl, l);
      nblk = __builtin_amdgcn_readlane(nb, l);
      ns = __builtin_amdgcn_readlane(n, l);
      r.win.s0 = c0;  // the window of lengths in hand (no second read)
      r.win.ctx_l = sq < S ? n : 0;
      found = true;
    }
  };
#pragma unroll
  for (int i = 0; i < kHeld; ++i)
    if (!found && i * kWave < S) try_window(i * kWave, held_n[i], held_incl[i]);
  if (!found) {
    int base = __builtin_amdgcn_readlane(held_incl[kHeld - 1], kWave - 1);
    for (int c0 = kHeld * kWave; c0 < S && !found; c0 += kWave) {
      const int n = c0 + lane < S ? decode_len(a, c0 + lane) : 0;
      const int incl = base + wave_incl_scan_i(seq_cost(c0 + lane < S ? blocks(n) : 0), lane);
      try_window(c0, n, incl);
      base = __builtin_amdgcn_readlane(incl, kWave - 1);
    }
  }
  const int L = nblk + c;
  const int h = (t - cum_s) / L;
  const int u = (t - cum_s) - h * L;
  r.j = u < c ? 0 : u - c;
  r.seg = StreamSeg{s, h, nblk, cum_s, ns - (nblk - 1) * kBlock};

  // count the wave's tiles: walk the segments its range touches
  SeqWindow win = r.win;
  StreamSeg sg = r.seg;
  int first = sg.cum + sg.h * (sg.nblk + c) + c + r.j;  // unit of the next tile
  int n = 0;
  for (;;) {
    const int seg_end = sg.cum + (sg.h + 1) * (sg.nblk + c);
    n += max(0, min(seg_end, tend) - first);
    if (seg_end >= tend || (sg.s >= S - 1 && sg.h == Hkv - 1)) break;
    if (++sg.h == Hkv) {
      sg.h = Hkv - 1;
      next_sequence(a, win, sg, lane);
    }
    first = sg.cum + sg.h * (sg.nblk + c) + c;
  }
  r.n = n;
  return n > 0;
}

// Step (sg, j) to the next tile of the tile order (one exists).
__device__ __forceinline__ void stream_step(const DecodeArgs &a, SeqWindow &win, StreamSeg &sg,
                                            int &j, int lane) {
  if (++j < sg.nblk) return;
  j = 0;
  if (++sg.h < a.num_kv_heads) return;
  sg.h = a.num_kv_heads - 1;
  next_sequence(a, win, sg, lane);
}

// True when one wave owns all of sg's tiles; piece = this wave's index among them.
__device__ __forceinline__ bool stream_single(const DecodeArgs &a, const StreamSeg &sg,
                                              const SplitGeom &sp, int w, int &piece) {
  const int first = sg.cum + sg.h * (sg.nblk + a.seg_cost) + a.seg_cost;  // first tile's unit
  const int wfirst = sp.wave_of(first), wlast = sp.wave_of(first + sg.nblk - 1);
  piece = w - wfirst;
  return wfirst == wlast;
}

// The wave's pipeline over its tiles, three stages deep: tile k is computed while
// tile k+1's K/V loads are in flight and tile k+2's block-table entry is being
// read.  Vector memory operations complete in issue order and the compiler waits
// on them by count, so inside the loop every load is issued unconditionally (the
// last tile is peeled off) and a segment's q is loaded before its first tile's
// K/V: a wait for one stage never drains the loads of the next.
// P (the per-dtype path) provides:
//   Tile; load(Tile&, tile index); compute(const Tile&, valid rows, masked);
//   prefetch_q(seg) into the next-q buffer; begin_segment() (next q becomes
//   current, state reset); emit(seg, single, piece).
template <class P>
__device__ __forceinline__ void stream_run(const DecodeArgs &a, P &path, int w, int lane) {
  StreamRange rg;
  if (!stream_range(a, w, lane, rg)) return;
  const int Hkv = a.num_kv_heads, n = rg.n;
  SeqWindow win = rg.win;
  const int sh = a.bs_shift;
  auto bt_of = [&](const StreamSeg &sg, int j) {
    return a.bt[(int64_t)sg.s * a.max_blocks_per_seq + (j >> sh)];
  };
  auto tile_of = [&](int bt, const StreamSeg &sg, int j) {
    return tile_index(__builtin_amdgcn_readfirstlane(bt), Hkv, sg.h, j, sh);
  };

  // stage 0 (compute): sg0, j0; stage 1 (loads in flight): sg1, j1, bt1
  StreamSeg sg0 = rg.seg, sg1 = rg.seg;
  int j0 = rg.j, j1 = rg.j;
  path.prefetch_q(sg0);
  const int bt0 = bt_of(sg0, j0);
  if (n > 1) stream_step(a, win, sg1, j1, lane);
  int bt1 = bt_of(sg1, j1);
  typename P::Tile tA, tB;
  path.load(tA, tile_of(bt0, sg0, j0), sg0, j0);
  path.begin_segment();

  // compute tile (sg0, j0); emit its segment when it ends there or the range does
  auto finish = [&](const typename P::Tile &cur, bool has_next) {
    const bool masked = j0 == sg0.nblk - 1 && sg0.tail < kBlock;
    path.compute(cur, masked ? sg0.tail : kBlock, masked);
    if (j0 == sg0.nblk - 1 || !has_next) {
      int piece;
      const bool single = stream_single(a, sg0, rg.sp, w, piece);
      path.emit(sg0, single, piece);
      if (has_next) path.begin_segment();
    }
  };
  // one step with a next tile: look up tile k+2, load tile k+1, compute tile k
  auto half = [&](int k, const typename P::Tile &cur, typename P::Tile &nxt) {
    StreamSeg sg2 = sg1;
    int j2 = j1;
    if (k + 2 < n) stream_step(a, win, sg2, j2, lane);
    const int bt2 = bt_of(sg2, j2);  // (a repeat of tile k+1's entry at the end)
    if (j1 == 0) path.prefetch_q(sg1);
    path.load(nxt, tile_of(bt1, sg1, j1), sg1, j1);
    finish(cur, true);
    sg0 = sg1;
    j0 = j1;
    sg1 = sg2;
    j1 = j2;
    bt1 = bt2;
  };
  for (int k = 0;;) {
    if (k + 1 >= n) {
      finish(tA, false);
      break;
    }
    half(k++, tA, tB);
    if (k + 1 >= n) {
      finish(tB, false);
      break;
    }
    half(k++, tB, tA);
  }
}

// Path for every (dtype, head_dim, group) but the MFMA one below: VALU dot products
// (v_dot2 for 16-bit keys) with the DPP reduce-scatter where the geometry allows.
template <int KV, int QT, int D, int G, bool NT>
struct GenericPath {
  using Gm = Geom<KV, D>;
  static constexpr int NL = Gm::NL, EPC = Gm::EPC, W32 = Gm::W32, LPT = Gm::LPT;
  static constexpr bool kFast = FastGeom<KV, D, G>::kOn;
  static constexpr bool kQuant = (KV == PA_FP8_E4M3 || KV == PA_I8);
  struct Tile {
    Chunk<W32> k[NL], v[NL];
    float ks, vs;
  };
  const DecodeArgs &a;
  const int lane, cidx, tg;
  const char *kbase, *vbase;
  DecodeState<KV, QT, D, G> st;
  FastState<KV, D, G> fs;
  QFrag<KV, EPC> qn[G];

  __device__ __forceinline__ GenericPath(const DecodeArgs &args, int ln)
      : a(args), lane(ln), cidx(ln % LPT), tg(ln / LPT),
        kbase(reinterpret_cast<const char *>(args.k) + ln * Gm::CB),
        vbase(reinterpret_cast<const char *>(args.v) + ln * Gm::CB) {}

  // Tile j of segment sg.  With a fused append (k_new set) the newest row of the
  // segment -- row tail - 1 of its last tile, not yet in the pool -- is read from
  // k_new / v_new instead; every load is still issued, only its address differs.
  __device__ __forceinline__ void load(Tile &t, int64_t tile, const StreamSeg &sg, int j) {
    const char *kp = kbase + tile * Gm::TILE_BYTES;
    const char *vp = vbase + tile * Gm::TILE_BYTES;
    const int nr = (a.k_new != nullptr && j == sg.nblk - 1) ? sg.tail - 1 : -1;
    const int64_t no = ((int64_t)sg.s * a.num_kv_heads + sg.h) * (D * Gm::E) + cidx * Gm::CB;
    const char *kn = reinterpret_cast<const char *>(a.k_new) + no;
    const char *vn = reinterpret_cast<const char *>(a.v_new) + no;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      t.k[i] = load_chunk<W32, NT>(i * Gm::TPI + tg == nr ? kn : kp + i * kWave * Gm::CB);
#pragma unroll
    for (int i = 0; i < NL; ++i)
      t.v[i] = load_chunk<W32, NT>(i * Gm::TPI + tg == nr ? vn : vp + i * kWave * Gm::CB);
    if constexpr (kQuant) {
      t.ks = a.k_scale[tile >> a.bs_shift];
      t.vs = a.v_scale[tile >> a.bs_shift];
    } else {
      t.ks = t.vs = 1.f;
    }
  }
  __device__ __forceinline__ void prefetch_q(const StreamSeg &sg) {
    const int64_t qbase = (decode_row(a, sg.s) * a.num_q_heads + sg.h * G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g) qn[g].template load<QT>(a.q, qbase + (int64_t)g * D + cidx * EPC);
  }
  __device__ __forceinline__ void begin_segment() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      st.q[g] = qn[g];
      st.m[g] = kNegBig;
      st.l[g] = 0.f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) st.acc[g][e] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < FastGeom<KV, D, G>::NVL; ++i) {
      fs.m[i] = kNegBig;
      fs.l[i] = 0.f;
    }
  }
  __device__ __forceinline__ void compute(const Tile &t, int valid, bool masked) {
    const float qs = kQuant ? a.qk_scale * t.ks : a.qk_scale;
    if constexpr (kFast) {
      if (masked)
        tile_update_fast<KV, QT, D, G, true>(st, fs, t.k, t.v, qs, t.vs, valid, tg, cidx);
      else
        tile_update_fast<KV, QT, D, G, false>(st, fs, t.k, t.v, qs, t.vs, kBlock, tg, cidx);
    } else {
      if (masked)
        tile_update<KV, QT, D, G, true>(st, t.k, t.v, qs, t.vs, valid, tg);
      else
        tile_update<KV, QT, D, G, false>(st, t.k, t.v, qs, t.vs, kBlock, tg);
    }
  }
  __device__ __forceinline__ void emit(const StreamSeg &sg, bool single, int piece) {
    if constexpr (kFast) fast_to_generic(st, fs);
    if constexpr (LPT == 16 && G % 4 == 0)
      emit_segment_rs<KV, QT, D, G>(a, st, sg.s, sg.h, single, piece, lane);
    else
      emit_segment<KV, QT, D, G>(a, st, sg.s, sg.h, single, piece, lane);
  }
};

template <int KV, int QT, int D, int G, bool NT>
__device__ __forceinline__ void decode_stream(const DecodeArgs &a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kDecodeWaves + threadIdx.x / kWave);
  GenericPath<KV, QT, D, G, NT> path(a, lane);
  stream_run(a, path, w, lane);
}

// ---- head_dim 64 and 128, GQA groups 2-8: both products of a tile on MFMA ----------
// Against the group's G query heads, one (block, kv head) tile of 16 keys x D dims
// gives two small dense products, run on matrix cores with the heads padded to 16:
//  * scores S^T[key][head] = K . Q^T on v_mfma_f32_16x16x32 (bf16, or f16 for f16
//    queries; the codes convert exactly), D/32 k-steps.  Lane (c16, g16) supplies
//    key row c16, dims mx_dim0(kk, g16) .. +7 of k-step kk (coalesced 16-byte loads)
//    and receives the scores of keys 4*g16 .. +3 for head c16;
//  * that is already the A-operand layout of O[head][dim] += P[head][key] . V[key][dim]
//    on v_mfma_f32_16x16x16 bf16 (row c16, keys 4*g16 .. +3): the probabilities
//    never leave the lane.  They enter with the tile's value scale folded in, split
//    as bf16 hi + lo (hi + lo matches p to about 2^-17 relative);
//  * the B operand (keys 4*g16 .. +3 of one dim) comes from four loads of value
//    rows 4*g16 + i, dims NE*c16 .. +NE-1 (NE = D/16), transposed inside the lane by
//    byte permutes and converted exactly to bf16; product e covers dims NE*c16 + e;
//  * lane (c16, g16) accumulates O rows 4*g16 + i (heads; rows G..15 are padding)
//    at dims NE*c16 + e.  Head c16's running max is the same in its four lanes; its
//    running sum is kept per lane over that lane's keys and summed at the end.
typedef _Float16 h8v_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8v_t __attribute__((ext_vector_type(8)));
typedef short s4v_t __attribute__((ext_vector_type(4)));
typedef float f4v_t __attribute__((ext_vector_type(4)));

// 16-bit pools (f16, bf16) take the same tile, where the VALU path's dot products
// and weighted sums per lane no longer keep up with the loads (Llama-3-70B-shaped
// decode, a group of 8 at D 128, on the VALU path: 147 us against 98 us at a group of
// 4 for the same K/V bytes): K enters the score product as stored; V is transposed by 16-bit
// permutes; for f16 pools the P.V product runs in f16 (P as f16 hi + lo, scaled by
// 2^10 so that small weights stay clear of f16's subnormals; the output takes the
// 2^-10 back), for bf16 pools in bf16 as for the codes.
// Workgroups per CU of the balanced-split stream kernels (either path): two where a
// wave's K+V tile is at most 4 KiB, i.e. 1-byte pools and 16-bit ones at head_dim
// 64 (more waves keep more of the small loads in flight), else one.
template <int KV, int D>
constexpr int stream_per_cu() {
  constexpr int E = KV == PA_F32 ? 4 : (KV == PA_F16 || KV == PA_BF16) ? 2 : 1;
  return 2 * kBlock * D * E <= 4096 ? 2 : 1;
}

template <int KV, int D, int G>
struct MxGeom {
  static constexpr bool k16 = KV == PA_F16 || KV == PA_BF16;
  static constexpr bool k8 = KV == PA_FP8_E4M3 || KV == PA_I8;
  // D 128: 1-byte pools at groups of 2, 4 and 8 (at 4 the VALU path's per-code
  // converts held fp8 to 3.3 TB/s); 16-bit pools at 4 and 8 (at 4 the tile's lighter
  // vector work leaves more of each wave's time to cover load latency: Llama-3-8B-
  // shaped decode 94.6 -> 92.8 us, prefix sharing 158.6 -> 143.9 us), not at 2, where
  // the two paths are level within a few percent either way.  D 64: both widths at
  // groups of 2, 4 and 8, where the VALU path's per-key work over half the bytes held
  // 16-bit pools to 2.8-4.6 TB/s and 1-byte pools to 1.2-2.7 TB/s.
  static constexpr bool kOn = D == 128   ? (k16 ? G >= 4 : (k8 && G >= 2))
                              : D == 64 ? ((k16 || k8) && G >= 2)
                                        : false;
  static constexpr int NE = D / 16;  // P.V products per tile: dims per lane
  static constexpr int KS = D / 32;  // k-steps of the score product
};
constexpr float kF16PScale = 1024.f;  // f16 pools: P enters the P.V product times 2^10

// Codes 2*HI and 2*HI + 1 of word w as two exact 16-bit values (T16 = PA_BF16 or
// PA_F16) packed in one word, the lower code in the low half.
template <int KV, int T16, bool HI>
__device__ __forceinline__ uint32_t codes2_to_16(uint32_t w) {
  if constexpr (KV == PA_FP8_E4M3) {
    if constexpr (T16 == PA_F16)
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.f, HI));
    else
      return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.f, HI));
  } else {
    const float f0 = (float)(int8_t)(w >> (HI ? 16 : 0));
    const float f1 = (float)(int8_t)(w >> (HI ? 24 : 8));
    if constexpr (T16 == PA_F16)
      return __builtin_bit_cast(uint32_t, h2_t{(_Float16)f0, (_Float16)f1});
    else
      return __builtin_bit_cast(uint32_t, bf2_t{(__bf16)f0, (__bf16)f1});
  }
}

// Two floats as a bf16 pair, each rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf2_t{(__bf16)x, (__bf16)y});
}

template <int QT>
__device__ __forceinline__ f4v_t mfma_qk(const u32x4 &a, const u32x4 &b, const f4v_t &c) {
  if constexpr (QT == PA_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8v_t, a),
                                                  __builtin_bit_cast(h8v_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8v_t, a),
                                                   __builtin_bit_cast(b8v_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f4v_t mfma_pv(const u32x2 &p, const u32x2 &v, const f4v_t &c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4v_t, p),
                                                   __builtin_bit_cast(s4v_t, v), c, 0, 0, 0);
}

// First of the 8 dims that lane group g16 supplies at k-step kk (same map for K and
// q): k-steps 2j and 2j + 1 cover dims [64j + 16*g16, +16).
__device__ __forceinline__ int mx_dim0(int kk, int g16) {
  return 64 * (kk >> 1) + 16 * g16 + 8 * (kk & 1);
}

// NW consecutive words at p (NW = 1, 2 or 4: one load).
template <int NW, bool NT>
__device__ __forceinline__ void load_words(uint32_t *w, const char *p) {
  if constexpr (NW == 4) {
    const u32x4 x = load_tile_part<u32x4, NT>(p);
    w[0] = x[0]; w[1] = x[1]; w[2] = x[2]; w[3] = x[3];
  } else if constexpr (NW == 2) {
    const u32x2 x = load_tile_part<u32x2, NT>(p);
    w[0] = x[0]; w[1] = x[1];
  } else {
    w[0] = load_tile_part<uint32_t, NT>(p);
  }
}

// One tile's operands in lane (c16, g16).
template <int D>
struct Q8Tile {
  u32x4 k[D / 64];         // key row c16: dims [64j + 16*g16, +16), k-steps 2j, 2j + 1
  uint32_t v[4][D / 64];   // value row 4*g16 + i: dims [(D/16)*c16, +D/16), one code a byte
  float ks, vs;            // the tile's K and V scales
};
template <int D>
struct Q16Tile {
  u32x4 k[D / 32];         // key row c16: dims mx_dim0(kk, g16) .. +7, the A operand of k-step kk
  uint32_t v[4][D / 32];   // value row 4*g16 + i: dims [(D/16)*c16, +D/16), two a word
};
template <int KV, int D>
using MxTileOf = std::conditional_t<MxGeom<KV, D, 8>::k16, Q16Tile<D>, Q8Tile<D>>;

template <int D>
struct MxAcc {
  f4v_t o[D / 16];  // o[e][i] = O[head 4*g16 + i][dim (D/16)*c16 + e]
  float m, l;       // head c16: running max (log2 units), this lane's running sum
};

// f16 P.V product (f16 pools)
__device__ __forceinline__ f4v_t mfma_pv_f16(const u32x2 &p, const u32x2 &v, const f4v_t &c) {
  typedef _Float16 h4v_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(h4v_t, p),
                                               __builtin_bit_cast(h4v_t, v), c, 0, 0, 0);
}

template <int KV, int QT, int D, bool MASK>
__device__ __forceinline__ void mx_tile(MxAcc<D> &st, const u32x4 *qb, const MxTileOf<KV, D> &t,
                                        float qk_scale, int valid_rows, int g16) {
  using Gm = MxGeom<KV, D, 8>;
  constexpr bool k16 = Gm::k16;
  constexpr int NE = Gm::NE, KS = Gm::KS;
  constexpr int T16 = QT == PA_F16 ? PA_F16 : PA_BF16;
  f4v_t sacc = f4v_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    u32x4 ka;
    if constexpr (k16) {
      ka = t.k[kk];  // as stored
    } else {
      const u32x4 &kw = t.k[kk >> 1];
      const uint32_t w0 = kw[2 * (kk & 1)], w1 = kw[2 * (kk & 1) + 1];
      ka[0] = codes2_to_16<KV, T16, false>(w0);
      ka[1] = codes2_to_16<KV, T16, true>(w0);
      ka[2] = codes2_to_16<KV, T16, false>(w1);
      ka[3] = codes2_to_16<KV, T16, true>(w1);
    }
    sacc = mfma_qk<QT>(ka, qb[kk], sacc);
  }
  float ks = 1.f, vs = KV == PA_F16 ? kF16PScale : 1.f;
  if constexpr (!k16) {
    ks = t.ks;
    vs = t.vs;
  }
  const float qs = qk_scale * ks;
  bool ok[4];
  float sv[4];
  float mx = kNegBig;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ok[i] = !MASK || 4 * g16 + i < valid_rows;
    sv[i] = ok[i] ? sacc[i] * qs : kNegBig;
    mx = fmaxf(mx, sv[i]);
  }
  mx = fmaxf(mx, xor_lanes<16>(mx));
  mx = fmaxf(mx, xor_lanes<32>(mx));
  const float mn = fmaxf(st.m, mx);
  if (__any(mn > st.m)) {
    const float alpha = fast_exp2(st.m - mn);
    st.l *= alpha;
    float ar[4];  // factors of this lane's O rows: heads 4*g16 + i live in lanes 4*g16 + i
#pragma unroll
    for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g16 + i, kWave);
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[e][i] *= ar[i];
  }
  st.m = mn;
  float pv[4];
  float psum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float p = fast_exp2(sv[i] - mn);
    if constexpr (MASK) p = ok[i] ? p : 0.f;
    psum += p;
    pv[i] = p * vs;
  }
  st.l += psum;
  u32x2 ph, pl;
  if constexpr (KV == PA_F16) {
    auto pack_h = [](float x, float y) { return __builtin_bit_cast(uint32_t, h2_t{(_Float16)x, (_Float16)y}); };
    ph[0] = pack_h(pv[0], pv[1]);
    ph[1] = pack_h(pv[2], pv[3]);
    pl[0] = pack_h(pv[0] - f16_lo(ph[0]), pv[1] - f16_hi(ph[0]));
    pl[1] = pack_h(pv[2] - f16_lo(ph[1]), pv[3] - f16_hi(ph[1]));
  } else {
    ph[0] = pack_bf16(pv[0], pv[1]);
    ph[1] = pack_bf16(pv[2], pv[3]);
    pl[0] = pack_bf16(pv[0] - bf16_lo(ph[0]), pv[1] - bf16_hi(ph[0]));
    pl[1] = pack_bf16(pv[2] - bf16_lo(ph[1]), pv[3] - bf16_hi(ph[1]));
  }
  if constexpr (k16) {
    // value rows past the context may hold anything (NaN included): zero their bits
    constexpr int NW = D / 32;
    uint32_t vr[4][NW];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int w = 0; w < NW; ++w) vr[i][w] = ok[i] ? t.v[i][w] : 0u;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      // keys 0..3 of dim NE*c16 + e: the low or high halves of word e/2 of the rows
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      u32x2 vb;
      vb[0] = __builtin_amdgcn_perm(vr[1][e >> 1], vr[0][e >> 1], sel);
      vb[1] = __builtin_amdgcn_perm(vr[3][e >> 1], vr[2][e >> 1], sel);
      if constexpr (KV == PA_F16) {
        st.o[e] = mfma_pv_f16(ph, vb, st.o[e]);
        st.o[e] = mfma_pv_f16(pl, vb, st.o[e]);
      } else {
        st.o[e] = mfma_pv(ph, vb, st.o[e]);
        st.o[e] = mfma_pv(pl, vb, st.o[e]);
      }
    }
    return;
  }

  // value rows past the context may hold anything (NaN included): zero their bits
  constexpr int NW = D / 64;
  uint32_t vr[4][NW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < NW; ++w) vr[i][w] = ok[i] ? t.v[i][w] : 0u;
#pragma unroll
  for (int c = 0; c < NW; ++c) {
    // bytes (r0.b, r1.b, ...) interleaved, then one word per dim: keys 0..3 of dim 4c + m
    const uint32_t t01l = __builtin_amdgcn_perm(vr[1][c], vr[0][c], 0x05010400u);
    const uint32_t t01h = __builtin_amdgcn_perm(vr[1][c], vr[0][c], 0x07030602u);
    const uint32_t t23l = __builtin_amdgcn_perm(vr[3][c], vr[2][c], 0x05010400u);
    const uint32_t t23h = __builtin_amdgcn_perm(vr[3][c], vr[2][c], 0x07030602u);
    uint32_t col[4];
    col[0] = __builtin_amdgcn_perm(t23l, t01l, 0x05040100u);
    col[1] = __builtin_amdgcn_perm(t23l, t01l, 0x07060302u);
    col[2] = __builtin_amdgcn_perm(t23h, t01h, 0x05040100u);
    col[3] = __builtin_amdgcn_perm(t23h, t01h, 0x07060302u);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      u32x2 vb;
      vb[0] = codes2_to_16<KV, PA_BF16, false>(col[m]);
      vb[1] = codes2_to_16<KV, PA_BF16, true>(col[m]);
      st.o[4 * c + m] = mfma_pv(ph, vb, st.o[4 * c + m]);
      st.o[4 * c + m] = mfma_pv(pl, vb, st.o[4 * c + m]);
    }
  }
}

// Write the wave's result for (s, kv head h): the normalised output when single,
// else the partial (m, l, acc) of `piece`.
template <int KV, int QT, int D, int G>
__device__ __forceinline__ void mx_emit(const DecodeArgs &a, const MxAcc<D> &st, int s, int h,
                                        bool single, int piece, int lane) {
  constexpr float kOut = KV == PA_F16 ? 1.f / kF16PScale : 1.f;  // undo the P scale of f16 pools
  constexpr int NE = D / 16;
  const int g16 = lane >> 4, c16 = lane & 15;
  float L = st.l;
  L += xor_lanes<16>(L);
  L += xor_lanes<32>(L);
  float mh[4], Lh[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    mh[i] = __shfl(st.m, 4 * g16 + i, kWave);
    Lh[i] = __shfl(L, 4 * g16 + i, kWave);
  }
  if (4 * g16 >= G) return;  // padding heads
  // the output row: by a scalar read for 16-bit pools; 1-byte pools have the next
  // tile's scales in flight as scalar loads, which that read's wait would drain
  int64_t qrow;
  if constexpr (MxGeom<KV, D, G>::k16)
    qrow = single ? decode_row_uniform(a, s) : 0;
  else
    qrow = decode_row(a, s);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (G < 4 && i >= G) break;
    const int64_t row = (int64_t)s * a.num_q_heads + h * G + 4 * g16 + i;      // workspace
    const int64_t orow = qrow * a.num_q_heads + h * G + 4 * g16 + i;          // output
    if (single) {
      const float inv = kOut / Lh[i];
      uint32_t pk[NE / 2];
#pragma unroll
      for (int e = 0; e < NE / 2; ++e) {
        const float x = st.o[2 * e][i] * inv, y = st.o[2 * e + 1][i] * inv;
        if constexpr (QT == PA_F16)
          pk[e] = __builtin_bit_cast(uint32_t, h2_t{(_Float16)x, (_Float16)y});
        else
          pk[e] = pack_bf16(x, y);
      }
      char *dst = reinterpret_cast<char *>(a.out) + (orow * D + NE * c16) * 2;
      if constexpr (NE == 8)
        *reinterpret_cast<u32x4 *>(dst) = u32x4{pk[0], pk[1], pk[2], pk[3]};
      else
        *reinterpret_cast<u32x2 *>(dst) = u32x2{pk[0], pk[1]};
    } else {
      const int64_t r = row * a.max_parts + piece;
      float *dst = a.ws_acc + r * D + NE * c16;
#pragma unroll
      for (int e4 = 0; e4 < NE / 4; ++e4)
        *reinterpret_cast<f4v_t *>(dst + 4 * e4) =
            f4v_t{st.o[4 * e4][i], st.o[4 * e4 + 1][i], st.o[4 * e4 + 2][i], st.o[4 * e4 + 3][i]} *
            kOut;
      if (c16 == 0) {
        a.ws_m[r] = mh[i];
        a.ws_l[r] = Lh[i];
      }
    }
  }
}

template <int KV, int QT, int D, int G, bool NT>
struct MxPath {
  using Gm = MxGeom<KV, D, G>;
  static constexpr bool k16 = Gm::k16;
  static constexpr int E = k16 ? 2 : 1, KS = Gm::KS, NE = Gm::NE, kTileBytes = kBlock * D * E;
  static constexpr int NWV = D * E / 64;  // words of a lane's value slice
  using Tile = MxTileOf<KV, D>;
  const DecodeArgs &a;
  const int lane, g16, c16;
  const char *kbase, *vbase;
  u32x4 qb[KS], qn[KS];  // B operand per k-step: q[head c16][8 dims]; qn: next segment's
  MxAcc<D> st;

  __device__ __forceinline__ MxPath(const DecodeArgs &args, int ln)
      : a(args), lane(ln), g16(ln >> 4), c16(ln & 15),
        kbase(reinterpret_cast<const char *>(args.k) + (ln & 15) * D * E + 16 * E * (ln >> 4)),
        vbase(reinterpret_cast<const char *>(args.v) + 4 * (ln >> 4) * D * E + NE * E * (ln & 15)) {}

  // Tile j of segment sg.  16-bit pools, with a fused append (k_new set): the
  // newest row of the segment -- row tail - 1 of its last tile, not yet in the pool
  // -- is read from k_new / v_new instead; every load is still issued, only its
  // address differs.  (1-byte pools take their new rows through the quantised
  // write before the decode.)
  __device__ __forceinline__ void load(Tile &t, int64_t tile, const StreamSeg &sg, int j) {
    if constexpr (k16) {
      const int nr = (a.k_new != nullptr && j == sg.nblk - 1) ? sg.tail - 1 : -1;
      const int64_t no = ((int64_t)sg.s * a.num_kv_heads + sg.h) * (D * E);
      const char *kn = reinterpret_cast<const char *>(a.k_new) + no + 16 * E * g16;
      const char *vn = reinterpret_cast<const char *>(a.v_new) + no + NE * E * c16;
      const char *kp = c16 == nr ? kn : kbase + tile * kTileBytes;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        t.k[kk] = load_tile_part<u32x4, NT>(kp + (mx_dim0(kk, 0)) * E);
      const char *vp = vbase + tile * kTileBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        load_words<NWV, NT>(t.v[i], 4 * g16 + i == nr ? vn : vp + i * D * E);
    } else {
      const char *kp = kbase + tile * kTileBytes;
#pragma unroll
      for (int j2 = 0; j2 < D / 64; ++j2) t.k[j2] = load_tile_part<u32x4, NT>(kp + 64 * j2);
      const char *vp = vbase + tile * kTileBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) load_words<NWV, NT>(t.v[i], vp + i * D);
      t.ks = a.k_scale[tile >> a.bs_shift];
      t.vs = a.v_scale[tile >> a.bs_shift];
    }
  }
  __device__ __forceinline__ void prefetch_q(const StreamSeg &sg) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qn[kk] = u32x4{0, 0, 0, 0};
    if (c16 < G) {
      const char *qp = reinterpret_cast<const char *>(a.q) +
                       ((decode_row(a, sg.s) * a.num_q_heads + sg.h * G + c16) * D) * 2;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        qn[kk] = *reinterpret_cast<const u32x4 *>(qp + mx_dim0(kk, g16) * 2);
    }
  }
  __device__ __forceinline__ void begin_segment() {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qb[kk] = qn[kk];
#pragma unroll
    for (int e = 0; e < NE; ++e) st.o[e] = f4v_t{0.f, 0.f, 0.f, 0.f};
    st.m = kNegBig;
    st.l = 0.f;
  }
  __device__ __forceinline__ void compute(const Tile &t, int valid, bool masked) {
    if (masked)
      mx_tile<KV, QT, D, true>(st, qb, t, a.qk_scale, valid, g16);
    else
      mx_tile<KV, QT, D, false>(st, qb, t, a.qk_scale, kBlock, g16);
  }
  __device__ __forceinline__ void emit(const StreamSeg &sg, bool single, int piece) {
    mx_emit<KV, QT, D, G>(a, st, sg.s, sg.h, single, piece, lane);
  }
};

template <int KV, int QT, int D, int G, bool NT>
__device__ __forceinline__ void decode_stream_mx(const DecodeArgs &a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(blockIdx.x * kDecodeWaves + threadIdx.x / kWave);
  MxPath<KV, QT, D, G, NT> path(a, lane);
  stream_run(a, path, w, lane);
}


// Fused append, after the decode has read the rows: store sequence s's new K and V
// row of kv head h at its slot, the pool position of token n - 1 ("5688vip" chapter
// 3, section 3.2: a new token's K/V goes at the end of the request's last block),
// slot = block_tables[s][(n - 1) / bs] * bs + (n - 1) % bs.  Lanes 0..31 move K,
// lanes 32..63 V, 16 bytes each (a row is at most 512 bytes).  Two halves, so that
// the caller can issue the row's load (which depends on nothing) together with its
// own first loads, and the table read with its second.
template <int D, int E>
__device__ __forceinline__ u32x4 append_load(const DecodeArgs &a, int s, int h, int lane) {
  constexpr int RB = D * E, CPR = RB / 16;
  static_assert(CPR <= 32, "row too wide");
  const int c = lane & 31;
  if (c >= CPR) return u32x4{0u, 0u, 0u, 0u};
  const int64_t src = ((int64_t)s * a.num_kv_heads + h) * RB + c * 16;
  return *reinterpret_cast<const u32x4 *>(
      reinterpret_cast<const char *>(lane >= 32 ? a.v_new : a.k_new) + src);
}
template <int D, int E>
__device__ __forceinline__ void append_store(const DecodeArgs &a, int s, int h, int n, int lane,
                                             const u32x4 &row) {
  constexpr int RB = D * E, CPR = RB / 16;
  const int bs = kBlock << a.bs_shift, p = n - 1;
  const int64_t blk = a.bt[(int64_t)s * a.max_blocks_per_seq + p / bs];
  const int64_t slot = blk * bs + p % bs;
  if (a.slots_out != nullptr && h == 0 && lane == 0) a.slots_out[s] = slot;
  const int c = lane & 31;
  if (c >= CPR) return;
  const int64_t dst = ((blk * a.num_kv_heads + h) * bs + p % bs) * RB + c * 16;
  *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(lane >= 32 ? a.pool_v : a.pool_k) + dst) = row;
}

// Second pass of the balanced split.  One wave per (sequence s, query head hq):
// lane p reads piece p's (m, l) (all pieces in flight at once), wave reductions
// give M = max_p m_p and L = sum_p 2^(m_p - M) l_p, then the pieces' acc rows come
// in 16-byte lane slices, several pieces per wave-wide load, and are combined as
//   out[d] = sum_p 2^(m_p - M) acc_p[d] / L.
// Nothing to do where one wave owned the whole segment (pieces == 1).
template <int QT, int D>
__device__ __forceinline__ void merge_stream(const DecodeArgs &a, int s, int hq, int lane) {
  // the split header and (fused append) the new K/V row, read beside the row's
  // length (all in bounds)
  const int h_t1 = a.hdr[0], h_t2 = a.hdr[1 + a.num_seqs], h_s = a.hdr[1 + s];
  const int G = a.num_q_heads / a.num_kv_heads;
  const int h = hq / G;
  const bool append = a.k_new != nullptr && hq % G == 0;
  u32x4 new_row = u32x4{0u, 0u, 0u, 0u};
  if (append) new_row = append_load<D, dtype_bytes(QT)>(a, s, h, lane);
  if (a.qsl != nullptr && a.qsl[s + 1] - a.qsl[s] != 1) return;  // not a decode row
  const int n = a.ctx[s];
  const int64_t o = (decode_row(a, s) * a.num_q_heads + hq) * D;
  if (n <= 0) {  // undefined input; keep the output finite and defined
    for (int d = lane; d < D; d += kWave) store_out<QT>(a.out, o + d, 0.f);
    if (a.slots_out != nullptr && hq == 0 && lane == 0) a.slots_out[s] = -1;
    return;
  }
  const int nblk = (n + kBlock - 1) / kBlock;
  // the split as stream_range made it
  const SplitGeom sp{h_t1, h_t2, a.skew > 0 ? a.num_waves / 2 : a.num_waves};
  const int seg0 = h_s + h * (nblk + a.seg_cost) + a.seg_cost;
  const int pieces = sp.wave_of(seg0 + nblk - 1) - sp.wave_of(seg0) + 1;
  if (pieces <= 1) {
    if (append) append_store<D, dtype_bytes(QT)>(a, s, h, n, lane, new_row);
    return;
  }
  const int64_t r0 = ((int64_t)s * a.num_q_heads + hq) * a.max_parts;
  // acc: each wave-wide load brings PPL whole pieces, lane l taking dims
  // 4*(l % LP) .. +3 of piece PPL*j + l / LP (16 bytes a lane), so the NB loads in
  // flight cover PPL*NB pieces (16 at D = 128): one round trip for the pieces of a
  // long context's segment instead of one per eight.
  constexpr int LP = D / 4, PPL = kWave / LP, NB = 8;
  static_assert(D % 4 == 0 && kWave % LP == 0, "head_dim splits into 16-byte lane slices");
  const int sub = lane / LP, dq = 4 * (lane % LP);
  // First batch of loads: (m, l) of every piece (lane p) and the acc of the first
  // PPL*NB pieces (the acc loads do not wait for the weights).
  float mp = kNegBig, lp = 0.f;
  if (lane < pieces) {
    mp = a.ws_m[r0 + lane];
    lp = a.ws_l[r0 + lane];
  }
  f4v_t v[NB];
  // (slots past the last piece are skipped by a uniform test: a segment of a short
  // context has two or three pieces)
  auto load_acc = [&](int p0) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (p0 + PPL * j >= pieces) break;
      const int p = p0 + PPL * j + sub;
      v[j] = p < pieces ? *reinterpret_cast<const f4v_t *>(a.ws_acc + (r0 + p) * D + dq)
                        : f4v_t{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_acc(0);
  // the append's table read goes out behind the pieces' loads
  if (append) append_store<D, dtype_bytes(QT)>(a, s, h, n, lane, new_row);
  float M = mp;
  for (int p = lane + kWave; p < pieces; p += kWave) M = fmaxf(M, a.ws_m[r0 + p]);
  M = fmaxf(M, xor_lanes<1>(M));
  M = fmaxf(M, xor_lanes<2>(M));
  M = fmaxf(M, dpp_f<kDppHalfMirror>(M));  // quads already agree: pairs quad 0 with quad 1
  M = fmaxf(M, xor_lanes<8>(M));
  M = fmaxf(M, xor_lanes<16>(M));
  M = fmaxf(M, xor_lanes<32>(M));
  float L = lane < pieces ? fast_exp2(mp - M) * lp : 0.f;
  for (int p = lane + kWave; p < pieces; p += kWave) L += fast_exp2(a.ws_m[r0 + p] - M) * a.ws_l[r0 + p];
  L = group_sum<64>(L);
  const float invL = 1.f / L;
  f4v_t acc = f4v_t{0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < pieces; p0 += PPL * NB) {
    if (p0 > 0) load_acc(p0);
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (p0 + PPL * j >= pieces) break;
      // weight of this lane's piece p: lane p holds its m when p < 64
      const int p = p0 + PPL * j + sub;
      const float mpj = __shfl(mp, p & (kWave - 1), kWave);
      const float mq = p < kWave ? mpj : (p < pieces ? a.ws_m[r0 + p] : kNegBig);
      const float wt = p < pieces ? fast_exp2(mq - M) : 0.f;
      acc += wt * v[j];
    }
  }
  // add up the PPL lane groups that hold the same dims
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (LP <= 16) acc[i] += xor_lanes<16>(acc[i]);
    acc[i] += xor_lanes<32>(acc[i]);
  }
  if (lane < LP) {
#pragma unroll
    for (int i = 0; i < 4; ++i) store_out<QT>(a.out, o + dq + i, acc[i] * invL);
  }
}

}  // namespace pa
