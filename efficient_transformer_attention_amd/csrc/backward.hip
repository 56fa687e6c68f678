// backward.hip — gradients of the FLASH layer for AMD Instinct MI355X (gfx950, CDNA4).
//
// The layer is the one of the forward (page "FLASH: Possibly the Most Interesting Efficient
// Transformer Design Recently", sections "Initial Power", "Weak Attention", "Mixed Chunk"); the
// page motivates the chunked form by its parallel training and prints no gradient, so the steps
// below are the chain rule of the forward's steps, in reverse order, for the loss Σ O ⊙ dO:
//
//   recompute  pack, proj (the gate's columns too; the pre-activations and V token-major), per-chunk scores P and the
//              exclusive prefix states S_g / n (the forward's own kernels)
//   mixb       per (chunk, value-column tile, token tile) two GEMMs into two accumulators:
//              V̂ᵀ = [V_gᵀ | S_gᵀ][P_g | Q_lin,g]ᵀ and dYᵀ = W_o dOᵀ; epilogue, with H_u = X W_u
//              from the recomputing projection: Y = U ⊙ V̂ (for dW_o), dV̂ = dY ⊙ U,
//              dH_u = dY ⊙ V̂ ⊙ SiLU'(H_u)
//   xpose      token-contiguous copies of X, dO and the heads (the weight gradients and the
//              per-chunk contractions over tokens read K-contiguous rows)
//   dscores    per chunk dW = dV̂ Vᵀ and A = Q_quad K_quadᵀ again: Pᵀ and dA = dW ⊙ 2 relu(A/c) / c
//              (masked); dQ_lin = dV̂ (S_g/n)ᵀ; and, in the same launch, the state gradients
//              dS_g = Q_lin,gᵀ dV̂_g / n summed over the LATER chunks (the forward's states and
//              carry kernels walking the chunks last to first)
//   dheads     dQ_quad = dA K_quad, dK_quad = dAᵀ Q_quad, dK_lin = V dTᵀ
//   dv         dVᵀ = [dV̂ᵀ | dTᵀ][Pᵀ | K_lin]ᵀ per chunk, times SiLU'(H_v)
//   dz         the rotary transpose, dZ = Σ γ_h dhead_h, dH_z, and partial sums for dγ, dβ
//   dx         dX = dH_u W_uᵀ + dH_v W_vᵀ + dH_z W_zᵀ (the input weights as stored)
//   wgrad      dW = Xᵀ dH and dW_o = Yᵀ dO, split over chunk ranges into fp32 partials
//   reduce     partial sums → dW_u, dW_v, dW_z, dW_o, dγ, dβ
//
// Every GEMM is the forward's TileGemm (K-contiguous operands straight into LDS, MFMA). Tiles are
// 128 x 128 with 8 waves for bf16 and 64 x 64 with 4 waves for fp32.

#include "kernels.h"

namespace {

template <class E> struct BShapes;
template <> struct BShapes<BF16> {
  static constexpr int BT = 128, WM = 2, WN = 4, NS = 2;
};
template <> struct BShapes<F32> {
  static constexpr int BT = 64, WM = 2, WN = 2, NS = 3;
};
// The backward's V̂ reads the recomputed P tile by tile like the forward's mix stage: its token
// tiles must be the scores stage's, or it could read causal P tiles that were never written.
static_assert(BShapes<BF16>::BT == Shapes<BF16>::kScoresBT && BShapes<F32>::BT == Shapes<F32>::kScoresBT,
              "backward tiles must match the scores tiles");

template <class E>
using BGemm = TileGemm<E, BShapes<E>::BT, BShapes<E>::BT, BShapes<E>::WM, BShapes<E>::WN,
                       BShapes<E>::NS>;

template <class E>
__device__ __forceinline__ int ksteps(int elems) {
  return (elems * E::kSize + kStageBytes - 1) / kStageBytes;
}

// Four consecutive elements as floats (8-byte aligned for bf16, 16-byte for fp32).
__device__ __forceinline__ void load4f(const uint16_t* p, float* o) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  o[0] = __uint_as_float(v[0] << 16);
  o[1] = __uint_as_float(v[0] & 0xFFFF0000u);
  o[2] = __uint_as_float(v[1] << 16);
  o[3] = __uint_as_float(v[1] & 0xFFFF0000u);
}
__device__ __forceinline__ void load4f(const float* p, float* o) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0];
  o[1] = v[1];
  o[2] = v[2];
  o[3] = v[3];
}

// ------------------------------------------------------------------------------ mixb
template <class E>
struct MixBArgs {
  using T = typename E::T;
  const T* Vt;   // [nbg, e, c]
  const T* St;   // causal [nbg, e, s], non-causal [B, e, s] (already / n)
  const T* P;    // [nbg, c, c]: P[i][j], query i, key j
  const T* Ql;   // [M, s]
  const T* Hu;   // [M, e]: X W_u before SiLU (the recomputing projection's)
  const T* Wo;   // [e, d], the input layout
  const T* dO;   // [M, d]
  T* Yt;         // [nbg, e, c]
  T* dVht;       // [nbg, e, c]
  T* dVhr;       // [M, e]
  T* dHut;       // [nbg, e, c]
  T* dHur;       // [M, e]
  int d, nbg, G, c, e, s, causal, lin;
};

template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void mixb_kernel(MixBArgs<E> p) {
  using G = BGemm<E>;
  using T = typename E::T;
  constexpr int BT = BShapes<E>::BT, WM = BShapes<E>::WM, WN = BShapes<E>::WN;
  __shared__ u32x4 lds[G::kLds];
  const int nte = (p.e + BT - 1) / BT;
  const int ntt = (p.c + BT - 1) / BT;
  const int lid = xcd_remap(blockIdx.x, p.nbg * nte * ntt);
  const int bg = lid / (nte * ntt);
  const int rem = lid % (nte * ntt);
  const int nt = rem / nte, mt = rem % nte;
  const int m0 = mt * BT, n0 = nt * BT;  // m: value column, n: token inside the chunk
  const int lane = threadIdx.x & 63, wave = wave_id();
  int wm, wn;
  balanced_wave<WM, WN>(wave, wm, wn);
  const int64_t tok0 = int64_t(bg) * p.c;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const int nkd = ksteps<E>(p.d);

  G gd;  // dYᵀ
  gd.zero();
  {
    const Src a = make_src(p.Wo, m0, p.d, E::kSize, p.e - m0, BT, p.d);
    const Src b = make_src(p.dO, tok0 + n0, p.d, E::kSize, p.c - n0, BT, p.d);
    gd.run(lds, nkd,
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = a;
             sb = b;
             ka = kb = t * kStageBytes;
           },
           NoPre(), wave, wm, wn, lane);
  }
  G g;  // V̂ᵀ, exactly as the forward's mix stage
  g.zero();
  {
    const int keys = p.causal ? min(p.c, n0 + BT) : p.c;
    const int nk0 = ksteps<E>(keys);
    const int nk1 = p.lin ? ksteps<E>(p.s) : 0;
    const Src a0 = make_src(p.Vt, int64_t(bg) * p.e + m0, p.c, E::kSize, p.e - m0, BT, p.c);
    const Src b0 = make_src(p.P, tok0 + n0, p.c, E::kSize, p.c - n0, BT, p.c);
    const Src a1 = make_src(p.St, slot * p.e + m0, p.s, E::kSize, p.e - m0, BT, p.s);
    const Src b1 = make_src(p.Ql, tok0 + n0, p.s, E::kSize, p.c - n0, BT, p.s);
    constexpr int kKeysPerTile = kStageBytes / E::kSize;
    const int last_token = n0 + (wn + 1) * G::WTN - 1;
    g.run(lds, nk0 + nk1,
          [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
            if (t < nk0) {
              sa = a0;
              sb = b0;
              ka = kb = t * kStageBytes;
            } else {
              sa = a1;
              sb = b1;
              ka = kb = (t - nk0) * kStageBytes;
            }
          },
          NoPre(), [&](int t) { return p.causal && t < nk0 && t * kKeysPerTile > last_token; },
          wave, wm, wn, lane);
  }

  // H_u of the lane's four value columns r.. of token column cl (tile-local), zeros off the edge
  auto load_hu = [&](int r, int cl, float* hu) {
    const int j = m0 + r, i = n0 + cl;
    if (j < p.e && i < p.c) {
      load4f(p.Hu + (tok0 + i) * p.e + j, hu);
    } else {
      hu[0] = hu[1] = hu[2] = hu[3] = 0.0f;
    }
  };
  // what: 0 Y = U ⊙ V̂, 1 dV̂ = dY ⊙ U, 2 dH_u = dY ⊙ V̂ ⊙ SiLU'(H_u)
  auto value = [&](int what, float hu, float dy, float vh) -> float {
    if (what == 0) return silu(hu) * vh;
    if (what == 1) return dy * silu(hu);
    return dy * vh * silu_grad(hu);
  };
  // token-contiguous (chunk-transposed) copies: Y, dV̂, dH_u
  T* const tdst[3] = {p.Yt, p.dVht, p.dHut};
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    g.template stage_cols<T>(
        lds, wave, wm, wn, lane,
        [&](int fi, int fj, int r, int cl, const f32x4& v, T* out) {
          float hu[4];
          load_hu(r, cl, hu);
#pragma unroll
          for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(value(w, hu[k], gd.acc[fi][fj][k], v[k]));
        },
        [&](int r, int cl, const u32x4& chunk) {
          const int j = m0 + r, i = n0 + cl;
          if (j < p.e && i < p.c)
            *reinterpret_cast<u32x4*>(tdst[w] + (int64_t(bg) * p.e + j) * p.c + i) = chunk;
        });
  }
  // token-major copies: dV̂, dH_u
  T* const rdst[2] = {p.dVhr, p.dHur};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    g.template stage_rows<T>(
        lds, wave, wm, wn, lane,
        [&](int fi, int fj, int r, int cl, const f32x4& v, T* out) {
          float hu[4];
          load_hu(r, cl, hu);
#pragma unroll
          for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(value(w + 1, hu[k], gd.acc[fi][fj][k], v[k]));
        },
        [&](int cl, int r, const u32x4& chunk) {
          const int j = m0 + r, i = n0 + cl;
          if (j < p.e && i < p.c) *reinterpret_cast<u32x4*>(rdst[w] + (tok0 + i) * p.e + j) = chunk;
        });
  }
}

// ------------------------------------------------------------------------------ xpose
// Batched transposes src[b] [R, C] -> dst[b] [C, R] in 64 x 64 tiles (as the weight packing).
template <class E>
struct XJob {
  const typename E::T* src;
  typename E::T* dst;
  int64_t sbs, dbs;  // batch strides, elements
  int R, C, tiles_c, tiles_per, first;
};
constexpr int kMaxXJobs = 8;
template <class E>
struct XArgs {
  XJob<E> job[kMaxXJobs];
  int njobs;
};

template <class E>
__global__ __launch_bounds__(256) void xpose_kernel(XArgs<E> args) {
  using T = typename E::T;
  constexpr int kPer16 = 16 / E::kSize;
  constexpr int kVecPerRow = 64 / kPer16;
  __shared__ T tile[64][64 + 1];
  const int bid = blockIdx.x;
  // job selection by unrolled selects (a dynamic index would copy the arguments to scratch)
  XJob<E> J = args.job[0];
#pragma unroll
  for (int i = 1; i < kMaxXJobs; ++i)
    if (i < args.njobs && bid >= args.job[i].first) J = args.job[i];
  int t = bid - J.first;
  const int b = t / J.tiles_per;
  t -= b * J.tiles_per;
  const int r0 = (t / J.tiles_c) * 64, c0 = (t % J.tiles_c) * 64;
  const T* src = J.src + b * J.sbs;
  T* dst = J.dst + b * J.dbs;
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 64 * kVecPerRow; idx += 256) {
    const int rr = idx / kVecPerRow, cv = (idx % kVecPerRow) * kPer16;
    if (r0 + rr < J.R && c0 + cv < J.C) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + int64_t(r0 + rr) * J.C + c0 + cv);
      const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
      for (int k = 0; k < kPer16; ++k) tile[rr][cv + k] = e[k];
    }
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * kVecPerRow; idx += 256) {
    const int cc = idx / kVecPerRow, rv = (idx % kVecPerRow) * kPer16;
    if (c0 + cc < J.C && r0 + rv < J.R) {
      u32x4 v;
      T* e = reinterpret_cast<T*>(&v);
#pragma unroll
      for (int k = 0; k < kPer16; ++k) e[k] = tile[rv + k][cc];
      *reinterpret_cast<u32x4*>(dst + int64_t(c0 + cc) * J.R + r0 + rv) = v;
    }
  }
}

template <class E>
struct XList {
  XArgs<E> a{};
  int tiles = 0;
  void add(const typename E::T* src, typename E::T* dst, int batch, int R, int C) {
    const int tr = int(cdiv(R, 64)), tc = int(cdiv(C, 64));
    XJob<E>& j = a.job[a.njobs++];
    j = {src, dst, int64_t(R) * C, int64_t(R) * C, R, C, tc, tr * tc, tiles};
    tiles += batch * tr * tc;
  }
  void launch(hipStream_t stream) {
    if (tiles == 0) return;
    for (int i = a.njobs; i < kMaxXJobs; ++i) a.job[i] = a.job[0];
    hipLaunchKernelGGL(xpose_kernel<E>, dim3(unsigned(tiles)), dim3(256), 0, stream, a);
  }
};

// ------------------------------------------------------------------------------ dscores
template <class E>
struct DScoresArgs {
  using T = typename E::T;
  const T* dVhr;  // [M, e]
  const T* Vr;    // [M, e]
  const T* Qq;    // [M, s]
  const T* Kq;    // [M, s]
  const T* Sr;    // [slots, s, e] (already / n)
  T* Pt;          // [nbg, c, c]: Pᵀ[j][i]
  T* dAr;         // [nbg, c, c]: dA[i][j]
  T* dAt;         // [nbg, c, c]: dA[j][i]
  float* dQl;     // [M, s]
  int nbg, G, c, s, e, causal;
  float inv_c;
};

// Tile (i-tile, j-tile) of one chunk: dW = dV̂ Vᵀ (over e) and A = Q_quad K_quadᵀ (over s);
// Pᵀ = relu(A/c)² and dA = dW ⊙ 2 relu(A/c) / c, zero above the diagonal when causal. Causal
// launches only the tiles on or below the diagonal; the consumers read no other.
template <class E>
__device__ __forceinline__ void dp_block(const DScoresArgs<E>& p, u32x4* lds, int bid) {
  using G = BGemm<E>;
  using T = typename E::T;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  const int ntc = (p.c + BT - 1) / BT;
  const int per_chunk = p.causal ? ntc * (ntc + 1) / 2 : ntc * ntc;
  const int lid = xcd_remap(bid, p.nbg * per_chunk);
  const int bg = lid / per_chunk;
  const int rem = lid % per_chunk;
  int it, jt;
  if (p.causal) {
    it = int((sqrtf(8.0f * float(rem) + 1.0f) - 1.0f) * 0.5f);
    while (it * (it + 1) / 2 > rem) --it;
    while ((it + 1) * (it + 2) / 2 <= rem) ++it;
    jt = rem - it * (it + 1) / 2;
  } else {
    it = rem / ntc;
    jt = rem % ntc;
  }
  const int i0 = it * BT, j0 = jt * BT;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tok0 = int64_t(bg) * p.c;

  G ga;
  ga.zero();
  {
    const Src a = make_src(p.Qq, tok0 + i0, p.s, E::kSize, p.c - i0, BT, p.s);
    const Src b = make_src(p.Kq, tok0 + j0, p.s, E::kSize, p.c - j0, BT, p.s);
    ga.run(lds, ksteps<E>(p.s),
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = a;
             sb = b;
             ka = kb = t * kStageBytes;
           },
           NoPre(), wave, wm, wn, lane);
  }
  G gp;
  gp.zero();
  {
    const Src a = make_src(p.dVhr, tok0 + i0, p.e, E::kSize, p.c - i0, BT, p.e);
    const Src b = make_src(p.Vr, tok0 + j0, p.e, E::kSize, p.c - j0, BT, p.e);
    gp.run(lds, ksteps<E>(p.e),
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = a;
             sb = b;
             ka = kb = t * kStageBytes;
           },
           NoPre(), wave, wm, wn, lane);
  }
  // what: 0 Pᵀ, 1 dA
  auto value = [&](int what, int fi, int fj, int k, int r, int cl) -> float {
    const int i = i0 + r + k, j = j0 + cl;
    if (p.causal && j > i) return 0.0f;
    const float x = fmaxf(ga.acc[fi][fj][k] * p.inv_c, 0.0f);
    return what == 0 ? x * x : gp.acc[fi][fj][k] * 2.0f * x * p.inv_c;
  };
  T* const base_t[2] = {p.Pt + tok0 * p.c, p.dAt + tok0 * p.c};
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    gp.template stage_rows<T>(
        lds, wave, wm, wn, lane,
        [&](int fi, int fj, int r, int cl, const f32x4&, T* out) {
#pragma unroll
          for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(value(w, fi, fj, k, r, cl));
        },
        [&](int cl, int r, const u32x4& chunk) {
          const int i = i0 + r, j = j0 + cl;
          if (i < p.c && j < p.c) *reinterpret_cast<u32x4*>(base_t[w] + int64_t(j) * p.c + i) = chunk;
        });
  }
  gp.template stage_cols<T>(
      lds, wave, wm, wn, lane,
      [&](int fi, int fj, int r, int cl, const f32x4&, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(value(1, fi, fj, k, r, cl));
      },
      [&](int r, int cl, const u32x4& chunk) {
        const int i = i0 + r, j = j0 + cl;
        if (i < p.c && j < p.c)
          *reinterpret_cast<u32x4*>(p.dAr + (tok0 + i) * p.c + j) = chunk;
      });
}

// A tile of rows (tokens of a chunk) x columns (s features) of a product over e, stored fp32
// row-major [M, s]: dQ_lin = dV̂ (S_g/n)ᵀ, and (in dheads) dK_lin = V dTᵀ.
template <class E>
__device__ __forceinline__ void rows_by_s_block(const typename E::T* A, const typename E::T* Bm,
                                                int64_t a_row0, int64_t b_row0, int a_rows,
                                                int b_rows, int K, float* out, int64_t out_row0,
                                                int f0, int s, u32x4* lds) {
  using G = BGemm<E>;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  G g;
  g.zero();
  const Src a = make_src(A, a_row0, K, E::kSize, a_rows, BT, K);
  const Src b = make_src(Bm, b_row0, K, E::kSize, b_rows, BT, K);
  g.run(lds, ksteps<E>(K),
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = b;
          ka = kb = t * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);
  g.template stage_cols<float>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, float* o) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
      },
      [&](int r, int cl, const u32x4& chunk) {
        if (r < a_rows && cl < b_rows)
          *reinterpret_cast<u32x4*>(out + (out_row0 + r) * s + f0 + cl) = chunk;
      });
}

template <class E>
__device__ __forceinline__ void dql_block(const DScoresArgs<E>& p, u32x4* lds, int bid) {
  constexpr int BT = BShapes<E>::BT;
  const int ntc = (p.c + BT - 1) / BT, nts = (p.s + BT - 1) / BT;
  const int lid = xcd_remap(bid, p.nbg * ntc * nts);
  const int bg = lid / (ntc * nts);
  const int rem = lid % (ntc * nts);
  const int it = rem / nts, rt = rem % nts;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const int64_t tok0 = int64_t(bg) * p.c + it * BT;
  rows_by_s_block<E>(p.dVhr, p.Sr, tok0, slot * p.s + rt * BT, p.c - it * BT, p.s - rt * BT, p.e,
                     p.dQl, tok0, rt * BT, p.s, lds);
}

// One launch, three roles by workgroup index: [0, n_dp) score-gradient tiles, [n_dp, n_dp +
// n_dql) dQ_lin tiles, then the state-gradient tiles (the forward's summaries walking the chunks
// last to first: Q_lin,gᵀ dV̂_g / n summed over the later chunks).
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dscores_states_kernel(
    DScoresArgs<E> p, int n_dp, int n_dql, StatesArgs<E> tp, int states_on) {
  using S = Shapes<E>;
  using GT = TileGemm<E, S::kStatesBM, S::kStatesBN, S::kStatesWM, S::kStatesWN, S::kStatesNS>;
  static_assert(GT::kThreads == BGemm<E>::kThreads, "all roles run with the same workgroup size");
  __shared__ u32x4 lds[BGemm<E>::kLds > GT::kLds ? BGemm<E>::kLds : GT::kLds];
  const int bid = blockIdx.x;
  if (bid < n_dp) {
    dp_block<E>(p, lds, bid);
  } else if (bid < n_dp + n_dql) {
    dql_block<E>(p, lds, bid - n_dp);
  } else if (states_on) {
    states_block<E, S::kStatesBM, S::kStatesBN, S::kStatesWM, S::kStatesWN, S::kStatesNS>(
        tp, lds, bid - n_dp - n_dql);
  }
}

// ------------------------------------------------------------------------------ dheads
template <class E>
struct DHeadsArgs {
  using T = typename E::T;
  const T* dAr;  // [nbg, c, c]
  const T* dAt;  // [nbg, c, c]
  const T* Kqt;  // [nbg, s, c]
  const T* Qqt;  // [nbg, s, c]
  const T* Vr;   // [M, e]
  const T* dTr;  // [slots, s, e] (already / n)
  float* dQq;    // [M, s]
  float* dKq;    // [M, s]
  float* dKl;    // [M, s]
  int nbg, G, c, s, e, causal;
};

// Role 0: dQ_quad = dA K_quad (rows i, K over keys j up to the tile's diagonal when causal).
// Role 1: dK_quad = dAᵀ Q_quad (rows j, K over queries i from the tile's diagonal when causal).
// Role 2: dK_lin = V dTᵀ (rows j, K over e).
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dheads_kernel(DHeadsArgs<E> p, int roles) {
  using G = BGemm<E>;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  __shared__ u32x4 lds[G::kLds];
  const int ntc = (p.c + BT - 1) / BT, nts = (p.s + BT - 1) / BT;
  const int per_role = p.nbg * ntc * nts;
  const int role = blockIdx.x / per_role;
  if (role >= roles) return;
  const int lid = xcd_remap(blockIdx.x - role * per_role, per_role);
  const int bg = lid / (ntc * nts);
  const int rem = lid % (ntc * nts);
  const int rt0 = rem / nts, st = rem % nts;
  const int r0 = rt0 * BT, f0 = st * BT;  // row tile (tokens of the chunk), feature tile
  const int64_t tok0 = int64_t(bg) * p.c;
  if (role == 2) {
    const int64_t slot = p.causal ? bg : bg / p.G;
    rows_by_s_block<E>(p.Vr, p.dTr, tok0 + r0, slot * p.s + f0, p.c - r0, p.s - f0, p.e, p.dKl,
                       tok0 + r0, f0, p.s, lds);
    return;
  }
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  // role 0 reads keys [0, min(c, r0 + BT)), role 1 queries [r0, c) when causal
  const int kbeg = (p.causal && role == 1) ? r0 : 0;
  const int kend = (p.causal && role == 0) ? min(p.c, r0 + BT) : p.c;
  const typename E::T* A = role == 0 ? p.dAr : p.dAt;
  const typename E::T* Bm = role == 0 ? p.Kqt : p.Qqt;
  G g;
  g.zero();
  const Src a = make_src(A, tok0 + r0, p.c, E::kSize, p.c - r0, BT, p.c);
  const Src b = make_src(Bm, int64_t(bg) * p.s + f0, p.c, E::kSize, p.s - f0, BT, p.c);
  const int kb0 = kbeg * E::kSize;
  g.run(lds, ksteps<E>(kend - kbeg),
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = b;
          ka = kb = kb0 + t * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);
  float* out = role == 0 ? p.dQq : p.dKq;
  g.template stage_cols<float>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, float* o) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
      },
      [&](int r, int cl, const u32x4& chunk) {
        const int i = r0 + r, f = f0 + cl;
        if (i < p.c && f < p.s) *reinterpret_cast<u32x4*>(out + (tok0 + i) * p.s + f) = chunk;
      });
}

// ------------------------------------------------------------------------------ dv
template <class E>
struct DVArgs {
  using T = typename E::T;
  const T* dVht;  // [nbg, e, c]
  const T* Pt;    // [nbg, c, c]: Pᵀ[j][i]
  const T* dTt;   // [slots, e, s] (already / n)
  const T* Klr;   // [M, s]
  const T* Hr;    // [M, e+s] pre-activations
  T* dHvr;        // [M, e]
  T* dHvt;        // [nbg, e, c]
  int nbg, G, c, s, e, causal, lin;
};

// Tile (value columns, keys j of a chunk): dVᵀ = dV̂ᵀ Pᵀᵀ over the queries i >= j (causal: from the
// tile's diagonal on) plus dTᵀ K_linᵀ over s; times SiLU'(H_v).
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dv_kernel(DVArgs<E> p) {
  using G = BGemm<E>;
  using T = typename E::T;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  __shared__ u32x4 lds[G::kLds];
  const int nte = (p.e + BT - 1) / BT, ntc = (p.c + BT - 1) / BT;
  const int lid = xcd_remap(blockIdx.x, p.nbg * nte * ntc);
  const int bg = lid / (nte * ntc);
  const int rem = lid % (nte * ntc);
  const int nt = rem / nte, mt = rem % nte;
  const int m0 = mt * BT, n0 = nt * BT;  // m: value column, n: key inside the chunk
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tok0 = int64_t(bg) * p.c;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const int kbeg = p.causal ? n0 : 0;
  const int nk0 = ksteps<E>(p.c - kbeg);
  const int nk1 = p.lin ? ksteps<E>(p.s) : 0;
  const Src a0 = make_src(p.dVht, int64_t(bg) * p.e + m0, p.c, E::kSize, p.e - m0, BT, p.c);
  const Src b0 = make_src(p.Pt, tok0 + n0, p.c, E::kSize, p.c - n0, BT, p.c);
  const Src a1 = make_src(p.dTt, slot * p.e + m0, p.s, E::kSize, p.e - m0, BT, p.s);
  const Src b1 = make_src(p.Klr, tok0 + n0, p.s, E::kSize, p.c - n0, BT, p.s);
  const int kb0 = kbeg * E::kSize;
  G g;
  g.zero();
  g.run(lds, nk0 + nk1,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          if (t < nk0) {
            sa = a0;
            sb = b0;
            ka = kb = kb0 + t * kStageBytes;
          } else {
            sa = a1;
            sb = b1;
            ka = kb = (t - nk0) * kStageBytes;
          }
        },
        NoPre(), wave, wm, wn, lane);
  // dH_v = dV ⊙ SiLU'(H_v), in place
  const int ncols = p.e + p.s;
  const int lr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < G::TM; ++i)
#pragma unroll
    for (int j = 0; j < G::TN; ++j) {
      const int col = m0 + wm * G::WTM + i * 16 + q * 4;  // first of four value columns
      const int key = n0 + wn * G::WTN + j * 16 + lr;
      if (col < p.e && key < p.c) {
        float h[4];
        load4f(p.Hr + (tok0 + key) * ncols + col, h);
#pragma unroll
        for (int k = 0; k < 4; ++k) g.acc[i][j][k] *= silu_grad(h[k]);
      }
    }
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int j = m0 + r, key = n0 + cl;
        if (j < p.e && key < p.c) *reinterpret_cast<u32x4*>(p.dHvr + (tok0 + key) * p.e + j) = chunk;
      });
  g.template stage_cols<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
      },
      [&](int r, int cl, const u32x4& chunk) {
        const int j = m0 + r, key = n0 + cl;
        if (j < p.e && key < p.c)
          *reinterpret_cast<u32x4*>(p.dHvt + (int64_t(bg) * p.e + j) * p.c + key) = chunk;
      });
}

// ------------------------------------------------------------------------------ dz
constexpr int kZRows = 32;  // token rows per dz workgroup (a multiple of 8)

template <class E>
struct DZArgs {
  using T = typename E::T;
  const float* dQq;  // [M, s]
  const float* dKq;
  const float* dQl;
  const float* dKl;
  const T* Hr;          // [M, e+s]; Z's pre-activations in columns e..
  const float* gamma;   // [4, s]
  T* dHzr;              // [M, s]
  T* dHzt;              // [nbg, s, c]
  float* gbpart;        // [nzb, 8, s]: rows 0..3 dγ, 4..7 dβ partial sums of workgroup row block
  int M, n, c, e, s, lin, rope;
  double log2_base;
};

// One thread per feature pair (2f, 2f+1) and group of rows; the rotary transpose turns a pair
// back by −m·θ. Rows go in runs of 8 tokens of one chunk so that dH_z's chunk-transposed copy
// leaves as 8-element runs.
template <class E>
__global__ __launch_bounds__(256) void dz_kernel(DZArgs<E> p) {
  using T = typename E::T;
  __shared__ float red[256][17];
  const int P = p.s / 2;
  const int pb = P > 256 ? 256 : P;  // pairs per workgroup
  const int RG = 256 / pb;           // row groups
  const int tid = threadIdx.x;
  const int pair = blockIdx.y * pb + tid % pb;
  const int rg = tid / pb;
  const bool act = rg < RG && pair < P;
  float acc[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) acc[k] = 0.0f;
  const int f0 = 2 * pair;
  if (act) {
    float gm[4][2];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      gm[h][0] = p.gamma[h * p.s + f0];
      gm[h][1] = p.gamma[h * p.s + f0 + 1];
    }
    const int ncols = p.e + p.s;
    const float* src[4] = {p.dQq, p.dKq, p.dQl, p.dKl};
    const int nheads = p.lin ? 4 : 2;
    const int row_end = min(p.M, int(blockIdx.x + 1) * kZRows);
    for (int rb = int(blockIdx.x) * kZRows + 8 * rg; rb < row_end; rb += 8 * RG) {
      alignas(16) T z0[8];
      alignas(16) T z1[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int row = rb + k;
        float g[4][2];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (h < nheads) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(src[h] + int64_t(row) * p.s + f0);
            g[h][0] = v[0];
            g[h][1] = v[1];
          } else {
            g[h][0] = g[h][1] = 0.0f;
          }
        }
        if (p.rope) {
          float cs, sn;
          rope_angle(row % p.n, rope_theta(f0, p.s, p.log2_base), &cs, &sn);
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            const float x0 = g[h][0], x1 = g[h][1];
            g[h][0] = rope_apply(x0, x1, f0, cs, -sn);
            g[h][1] = rope_apply(x1, x0, f0 + 1, cs, -sn);
          }
        }
        const T* hz = p.Hr + int64_t(row) * ncols + p.e + f0;
        const float hz0 = to_f32(hz[0]), hz1 = to_f32(hz[1]);
        const float zz[2] = {silu(hz0), silu(hz1)};
        float dz0 = 0.0f, dz1 = 0.0f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          dz0 = fmaf(gm[h][0], g[h][0], dz0);
          dz1 = fmaf(gm[h][1], g[h][1], dz1);
          acc[h * 2] = fmaf(zz[0], g[h][0], acc[h * 2]);
          acc[h * 2 + 1] = fmaf(zz[1], g[h][1], acc[h * 2 + 1]);
          acc[8 + h * 2] += g[h][0];
          acc[8 + h * 2 + 1] += g[h][1];
        }
        const float d0 = dz0 * silu_grad(hz0), d1 = dz1 * silu_grad(hz1);
        T* o = p.dHzr + int64_t(row) * p.s + f0;
        o[0] = from_f32<E>(d0);
        o[1] = from_f32<E>(d1);
        z0[k] = from_f32<E>(d0);
        z1[k] = from_f32<E>(d1);
      }
      const int64_t bg = rb / p.c, t = rb % p.c;  // 8 rows inside one chunk (c % 8 == 0)
      T* o0 = p.dHzt + (bg * p.s + f0) * p.c + t;  // 16-byte aligned: t and c are multiples of 8
      T* o1 = o0 + p.c;
      constexpr int kVec = 16 / int(sizeof(T));
#pragma unroll
      for (int v = 0; v < 8 / kVec; ++v) {
        *reinterpret_cast<u32x4*>(o0 + v * kVec) = *reinterpret_cast<const u32x4*>(z0 + v * kVec);
        *reinterpret_cast<u32x4*>(o1 + v * kVec) = *reinterpret_cast<const u32x4*>(z1 + v * kVec);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) red[tid][k] = acc[k];
  __syncthreads();
  if (act && rg == 0) {
    for (int r = 1; r < RG; ++r)
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] += red[tid + r * pb][k];
    float* out = p.gbpart + int64_t(blockIdx.x) * 8 * p.s;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      out[h * p.s + f0] = acc[h * 2];
      out[h * p.s + f0 + 1] = acc[h * 2 + 1];
      out[(4 + h) * p.s + f0] = acc[8 + h * 2];
      out[(4 + h) * p.s + f0 + 1] = acc[8 + h * 2 + 1];
    }
  }
}

// ------------------------------------------------------------------------------ dx
template <class E>
struct DXArgs {
  using T = typename E::T;
  const T* Wu;    // [d, e]
  const T* Wv;    // [d, e]
  const T* Wz;    // [d, s]
  const T* dHur;  // [M, e]
  const T* dHvr;  // [M, e]
  const T* dHzr;  // [M, s]
  T* dX;          // [M, d]
  int M, d, e, s;
};

// dXᵀ tiles (input features x tokens) over the three K ranges e | e | s.
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dx_kernel(DXArgs<E> p) {
  using G = BGemm<E>;
  using T = typename E::T;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  __shared__ u32x4 lds[G::kLds];
  const int ntd = (p.d + BT - 1) / BT, ntt = (p.M + BT - 1) / BT;
  const int lid = xcd_remap(blockIdx.x, ntd * ntt);
  const int nt = lid / ntd, mt = lid % ntd;
  const int m0 = mt * BT, n0 = nt * BT;  // m: input feature, n: token
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  const int nke = ksteps<E>(p.e), nks = ksteps<E>(p.s);
  const Src au = make_src(p.Wu, m0, p.e, E::kSize, p.d - m0, BT, p.e);
  const Src av = make_src(p.Wv, m0, p.e, E::kSize, p.d - m0, BT, p.e);
  const Src az = make_src(p.Wz, m0, p.s, E::kSize, p.d - m0, BT, p.s);
  const Src bu = make_src(p.dHur, n0, p.e, E::kSize, p.M - n0, BT, p.e);
  const Src bv = make_src(p.dHvr, n0, p.e, E::kSize, p.M - n0, BT, p.e);
  const Src bz = make_src(p.dHzr, n0, p.s, E::kSize, p.M - n0, BT, p.s);
  G g;
  g.zero();
  g.run(lds, 2 * nke + nks,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          if (t < nke) {
            sa = au;
            sb = bu;
            ka = kb = t * kStageBytes;
          } else if (t < 2 * nke) {
            sa = av;
            sb = bv;
            ka = kb = (t - nke) * kStageBytes;
          } else {
            sa = az;
            sb = bz;
            ka = kb = (t - 2 * nke) * kStageBytes;
          }
        },
        NoPre(), wave, wm, wn, lane);
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int k = m0 + r, i = n0 + cl;
        if (k < p.d && i < p.M) *reinterpret_cast<u32x4*>(p.dX + int64_t(i) * p.d + k) = chunk;
      });
}

// ------------------------------------------------------------------------------ wgrad
// out[q] [Fa, Fb] = Σ over the tokens of chunks [q cps, (q+1) cps) of A[chunk] [Fa, c] ·
// B[chunk] [Fb, c]ᵀ: operands chunk-transposed (token-contiguous), fp32 partial per split q.
template <class E>
struct WJob {
  const typename E::T* A;
  const typename E::T* B;
  float* out;
  int Fa, Fb, tiles_m, tiles_n, first;
};
template <class E>
struct WArgs {
  WJob<E> job[4];
  int njobs, nbg, c, cps, splits;
};

template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void wgrad_kernel(WArgs<E> p, int total) {
  using G = BGemm<E>;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  __shared__ u32x4 lds[G::kLds];
  const int lid = xcd_remap(blockIdx.x, total);
  WJob<E> J = p.job[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < p.njobs && lid >= p.job[i].first) J = p.job[i];
  int t = lid - J.first;
  const int per_split = J.tiles_m * J.tiles_n;
  const int q = t / per_split;
  t -= q * per_split;
  const int nt = t / J.tiles_m, mt = t % J.tiles_m;
  const int m0 = mt * BT, n0 = nt * BT;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  const int cbeg = q * p.cps;
  const int nch = min(p.nbg, cbeg + p.cps) - cbeg;
  const int nkc = ksteps<E>(p.c);
  G g;
  g.zero();
  g.run(lds, nch * nkc,
        [&](int tt, Src& sa, int& ka, Src& sb, int& kb) {
          const int64_t chunk = cbeg + tt / nkc;
          sa = make_src(J.A, chunk * J.Fa + m0, p.c, E::kSize, J.Fa - m0, BT, p.c);
          sb = make_src(J.B, chunk * J.Fb + n0, p.c, E::kSize, J.Fb - n0, BT, p.c);
          ka = kb = (tt % nkc) * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);
  float* out = J.out + int64_t(q) * J.Fa * J.Fb;
  g.template stage_cols<float>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, float* o) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
      },
      [&](int r, int cl, const u32x4& chunk) {
        const int row = m0 + r, col = n0 + cl;
        if (row < J.Fa && col < J.Fb)
          *reinterpret_cast<u32x4*>(out + int64_t(row) * J.Fb + col) = chunk;
      });
}

// ------------------------------------------------------------------------------ reduce
template <class E>
struct RJob {
  const float* part;    // [splits, count]
  typename E::T* out;   // [count]
  int64_t count4;       // count / 4
  int64_t first4;       // first quad of this job in the launch
};
template <class E>
struct RArgs {
  RJob<E> job[4];
  int njobs, splits;
};

template <class E>
__global__ __launch_bounds__(256) void wreduce_kernel(RArgs<E> p, int64_t total4) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= total4) return;
  RJob<E> J = p.job[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < p.njobs && idx >= p.job[i].first4) J = p.job[i];
  const int64_t i4 = idx - J.first4;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < p.splits; ++q) {
    const f32x4 v = reinterpret_cast<const f32x4*>(J.part)[int64_t(q) * J.count4 + i4];
    s[0] += v[0];
    s[1] += v[1];
    s[2] += v[2];
    s[3] += v[3];
  }
  store4(J.out + i4 * 4, s[0], s[1], s[2], s[3]);
}

// dγ, dβ [4, s] each from the dz partials [nzb, 8, s]: 16 outputs per workgroup, 64 lanes per
// output each summing every 64th partial (four loads in flight), then a fixed-order sum of the 64.
__global__ __launch_bounds__(1024) void gbreduce_kernel(const float* gbpart, int nzb, int s,
                                                       float* dgamma, float* dbeta) {
  __shared__ float red[64][16 + 1];
  const int o = threadIdx.x & 15, l = threadIdx.x >> 4;
  const int j = blockIdx.x * 16 + o;  // output index in [0, 8 s)
  const int64_t stride = int64_t(8) * s;
  float v = 0.0f;
  if (j < 8 * s) {
    int b = l;
    for (; b + 192 < nzb; b += 256) {
      const float x0 = gbpart[int64_t(b) * stride + j], x1 = gbpart[int64_t(b + 64) * stride + j];
      const float x2 = gbpart[int64_t(b + 128) * stride + j], x3 = gbpart[int64_t(b + 192) * stride + j];
      v += (x0 + x1) + (x2 + x3);
    }
    for (; b < nzb; b += 64) v += gbpart[int64_t(b) * stride + j];
  }
  red[l][o] = v;
  __syncthreads();
  if (l == 0 && j < 8 * s) {
    for (int k = 1; k < 64; ++k) v += red[k][o];
    if (j < 4 * s)
      dgamma[j] = v;
    else
      dbeta[j - 4 * s] = v;
  }
}

// zero-fill (gradients of an empty batch), a kernel rather than a memset so that the whole
// backward can be captured in a graph
__global__ __launch_bounds__(256) void zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += int64_t(gridDim.x) * 256)
    p[i] = 0u;
}

// ------------------------------------------------------------------------------ host plan
enum BRegion {
  BR_HU, BR_HR, BR_VR, BR_XT, BR_DOT, BR_QQT, BR_KQT, BR_QLT, BR_KLR, BR_SR, BR_YT, BR_DVHT, BR_DVHR,
  BR_DHUT, BR_DHUR, BR_PT, BR_DAR, BR_DAT, BR_DTT, BR_DCARRY, BR_DTR, BR_DQQ, BR_DKQ, BR_DQL,
  BR_DKL, BR_DHVR, BR_DHVT, BR_DHZR, BR_DHZT, BR_WPART, BR_GBPART, BR_COUNT
};

struct BPlan {
  Plan f;                 // the forward's regions come first in the workspace
  int64_t slots;          // state slots: chunks (causal) or sequences
  int64_t splits, cps;    // weight gradients: chunk-range splits, chunks per split
  int64_t wcount[4];      // elements of dW_u, dW_v, dW_z, dW_o
  int64_t nzb;            // dz row blocks
  int64_t bt;             // backward tile
  size_t off[BR_COUNT];
  size_t total;
};

constexpr int64_t kWgradTargetBlocks = 2048;

int make_bplan(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk, int causal,
               flashgau_dtype dtype, BPlan* bp) {
  memset(bp, 0, sizeof(*bp));
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &bp->f);
  if (rc != FLASHGAU_OK) return rc;
  const Plan& f = bp->f;
  bp->wcount[0] = bp->wcount[1] = d * e;
  bp->wcount[2] = d * s;
  bp->wcount[3] = e * d;
  if (f.M == 0) {
    bp->total = 0;
    return FLASHGAU_OK;
  }
  const int64_t M = f.M, nbg = f.nbg;
  bp->bt = dtype == FLASHGAU_BF16 ? BShapes<BF16>::BT : BShapes<F32>::BT;
  const int64_t bt = bp->bt;
  bp->slots = causal ? nbg : B;
  const int64_t tiles_per_split = 2 * cdiv(d, bt) * cdiv(e, bt) + cdiv(d, bt) * cdiv(s, bt) +
                                  cdiv(e, bt) * cdiv(d, bt);
  int64_t splits = std::max<int64_t>(1, std::min<int64_t>(nbg, cdiv(kWgradTargetBlocks, tiles_per_split)));
  bp->cps = cdiv(nbg, splits);
  bp->splits = cdiv(nbg, bp->cps);
  bp->nzb = cdiv(M, kZRows);
  const int64_t esz = f.esz;
  int64_t cnt[BR_COUNT], sz[BR_COUNT];
  for (int i = 0; i < BR_COUNT; ++i) sz[i] = esz;
  int64_t t0;
  if (!mul_ok(M, e + s, &cnt[BR_HR])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(M, e, &cnt[BR_VR])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_HU] = cnt[BR_VR];
  if (!mul_ok(M, d, &cnt[BR_XT])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_DOT] = cnt[BR_XT];
  if (!mul_ok(M, s, &cnt[BR_QQT])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_KQT] = cnt[BR_QLT] = cnt[BR_KLR] = cnt[BR_QQT];
  if (!mul_ok(bp->slots, s, &t0) || !mul_ok(t0, e, &cnt[BR_SR])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_YT] = cnt[BR_DVHT] = cnt[BR_DVHR] = cnt[BR_DHUT] = cnt[BR_DHUR] = cnt[BR_VR];
  if (!mul_ok(M, chunk, &cnt[BR_PT])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_DAR] = cnt[BR_DAT] = cnt[BR_PT];
  cnt[BR_DTT] = cnt[BR_DTR] = cnt[BR_SR];
  if (!mul_ok(B * f.ng, e, &t0) || !mul_ok(t0, s, &cnt[BR_DCARRY])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_DQQ] = cnt[BR_DKQ] = cnt[BR_DQL] = cnt[BR_DKL] = cnt[BR_QQT];
  sz[BR_DQQ] = sz[BR_DKQ] = sz[BR_DQL] = sz[BR_DKL] = 4;
  cnt[BR_DHVR] = cnt[BR_DHVT] = cnt[BR_VR];
  cnt[BR_DHZR] = cnt[BR_DHZT] = cnt[BR_QQT];
  const int64_t wtot = bp->wcount[0] + bp->wcount[1] + bp->wcount[2] + bp->wcount[3];
  if (!mul_ok(bp->splits, wtot, &cnt[BR_WPART])) return FLASHGAU_ERR_BAD_SHAPE;
  sz[BR_WPART] = 4;
  cnt[BR_GBPART] = bp->nzb * 8 * s;
  sz[BR_GBPART] = 4;
  size_t off = (f.total + 255) & ~size_t(255);
  for (int i = 0; i < BR_COUNT; ++i) {
    int64_t bytes;
    if (!mul_ok(cnt[i], sz[i], &bytes)) return FLASHGAU_ERR_BAD_SHAPE;
    bp->off[i] = off;
    const size_t padded = (size_t(bytes) + 255) & ~size_t(255);
    if (__builtin_add_overflow(off, padded, &off)) return FLASHGAU_ERR_BAD_SHAPE;
  }
  bp->total = off;
  // grid sizes
  const int64_t ntc = cdiv(chunk, bt), nts = cdiv(s, bt), nte = cdiv(e, bt);
  const int64_t xtiles = 2 * nbg * cdiv(chunk, 64) * cdiv(d, 64) + 4 * nbg * cdiv(chunk, 64) * cdiv(s, 64) +
                         bp->slots * cdiv(e, 64) * cdiv(s, 64);
  const int64_t grids[] = {
      nbg * nte * ntc,                                                           // mixb, dv
      xtiles,                                                                    // xpose
      nbg * ntc * ntc + nbg * ntc * nts + B * f.ng * cdiv(s, kStatesTileM) * cdiv(e, kStatesTileN),
      3 * nbg * ntc * nts,                                                       // dheads
      cdiv(d, bt) * cdiv(M, bt),                                                 // dx
      bp->splits * tiles_per_split,                                              // wgrad
      cdiv(wtot / 4, 256),                                                       // reduce
      bp->nzb * cdiv(s / 2, 256),                                                // dz
  };
  for (int64_t g : grids)
    if (g > kMaxBlocks) return FLASHGAU_ERR_BAD_SHAPE;
  return FLASHGAU_OK;
}

// ------------------------------------------------------------------------------ launches
template <class E>
int launch_backward(const BPlan& bp, const void* X, const void* W_u, const void* W_v,
                    const void* W_z, const float* gamma, const float* beta, const void* W_o,
                    const void* dO, int causal, float rope_base, void* dX, void* dW_u, void* dW_v,
                    void* dW_z, float* dgamma, float* dbeta, void* dW_o, char* ws,
                    hipStream_t stream) {
  using T = typename E::T;
  using S = Shapes<E>;
  constexpr int kThreads = BGemm<E>::kThreads;
  const Plan& pl = bp.f;
  auto W = [&](int r) { return reinterpret_cast<T*>(ws + pl.off[r]); };
  auto R = [&](int r) { return reinterpret_cast<T*>(ws + bp.off[r]); };
  auto Rf = [&](int r) { return reinterpret_cast<float*>(ws + bp.off[r]); };
  T *WcatT = W(FLASHGAU_WS_WCAT_T), *WoT = W(FLASHGAU_WS_WO_T), *Vt = W(FLASHGAU_WS_VT);
  T *Qq = W(FLASHGAU_WS_QQ), *Kq = W(FLASHGAU_WS_KQ), *Ql = W(FLASHGAU_WS_QL);
  T *Klt = W(FLASHGAU_WS_KLT), *P = W(FLASHGAU_WS_P), *St = W(FLASHGAU_WS_ST);
  T* Carry = W(FLASHGAU_WS_CARRY);
  const T* Xp = reinterpret_cast<const T*>(X);
  const T* dOp = reinterpret_cast<const T*>(dO);
  const int M = int(pl.M), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);
  const int nbg = int(pl.nbg), G = int(pl.G), B = int(pl.B);
  const int bt = int(bp.bt);
  const bool lin = !(causal && pl.G == 1);
  const int rope = rope_base > 0.0f ? 1 : 0;
  const double log2_base = rope ? log2(double(rope_base)) : 0.0;
  const float inv_n = float(1.0 / double(pl.n));

  // ---- recompute the forward's intermediates
  launch_pack<E>(W_u, W_v, W_z, W_o, d, e, s, WcatT, WoT, stream);
  {
    ProjArgs<E> a{Xp, WcatT, Vt, Qq, Kq, Ql, Klt, gamma, beta, M, d, e, s, c,
                  int(pl.n), rope, log2_base, R(BR_HR), R(BR_VR), R(BR_HU)};
    const int64_t nb = cdiv(M, S::kProjBM) * cdiv(2 * e + s, S::kProjBN);
    hipLaunchKernelGGL(
        (proj_kernel<E, S::kProjBM, S::kProjBN, S::kProjWM, S::kProjWN, S::kProjNS, true>),
        dim3(unsigned(nb)), dim3(64 * S::kProjWM * S::kProjWN), 0, stream, a);
  }
  {
    ScoresArgs<E> sa{Qq, Kq, P, nbg, c, s, causal, 1.0f / float(c)};
    const int64_t ntc = cdiv(c, S::kScoresBT);
    const int64_t nsb = pl.nbg * (causal ? ntc * (ntc + 1) / 2 : ntc * ntc);
    const int64_t nsb8 = cdiv(nsb, kXcds) * kXcds;
    StatesArgs<E> ta{Klt, Vt, St, Carry, B, G, s, e, c, causal, int(pl.ng), int(pl.gs), inv_n, 0};
    const int64_t ntb = lin ? pl.B * pl.ng * cdiv(s, S::kStatesBM) * cdiv(e, S::kStatesBN) : 0;
    hipLaunchKernelGGL((scores_states_kernel<E, S>), dim3(unsigned(nsb8 + ntb)),
                       dim3(64 * S::kScoresWM * S::kScoresWN), 0, stream, sa, int(nsb8), int(nsb), ta,
                       int(lin));
  }
  if (lin && pl.ng > 1) {
    CarryArgs<E> a{St, Carry, B, G, int(pl.ng), int(pl.gs), causal, int64_t(e) * s, 0};
    hipLaunchKernelGGL(carry_kernel<E>, dim3(unsigned(cdiv(pl.B * e * s / 8, 256))), dim3(256), 0,
                       stream, a);
  }

  // ---- gate, output projection and V̂
  {
    MixBArgs<E> a{Vt, St, P, Ql, R(BR_HU), reinterpret_cast<const T*>(W_o), dOp, R(BR_YT),
                  R(BR_DVHT), R(BR_DVHR), R(BR_DHUT), R(BR_DHUR), d, nbg, G, c, e, s, causal,
                  int(lin)};
    const int64_t nb = pl.nbg * cdiv(e, bt) * cdiv(c, bt);
    hipLaunchKernelGGL(mixb_kernel<E>, dim3(unsigned(nb)), dim3(kThreads), 0, stream, a);
  }
  // ---- token-contiguous copies
  {
    XList<E> xl;
    xl.add(Xp, R(BR_XT), nbg, c, d);
    xl.add(dOp, R(BR_DOT), nbg, c, d);
    xl.add(Qq, R(BR_QQT), nbg, c, s);
    xl.add(Kq, R(BR_KQT), nbg, c, s);
    xl.add(Ql, R(BR_QLT), nbg, c, s);
    xl.add(Klt, R(BR_KLR), nbg, s, c);
    if (lin) xl.add(St, R(BR_SR), int(bp.slots), e, s);
    xl.launch(stream);
  }
  // ---- score gradients, dQ_lin, state gradients
  {
    DScoresArgs<E> a{R(BR_DVHR), R(BR_VR), Qq, Kq, R(BR_SR), R(BR_PT), R(BR_DAR), R(BR_DAT),
                     Rf(BR_DQL), nbg, G, c, s, e, causal, 1.0f / float(c)};
    const int64_t ntc = cdiv(c, bt), nts = cdiv(s, bt);
    const int64_t n_dp = pl.nbg * (causal ? ntc * (ntc + 1) / 2 : ntc * ntc);
    const int64_t n_dql = lin ? pl.nbg * ntc * nts : 0;
    StatesArgs<E> ta{R(BR_QLT), R(BR_DVHT), R(BR_DTT), R(BR_DCARRY), B, G, s, e, c, causal,
                     int(pl.ng), int(pl.gs), inv_n, 1};
    const int64_t ntb = lin ? pl.B * pl.ng * cdiv(s, S::kStatesBM) * cdiv(e, S::kStatesBN) : 0;
    hipLaunchKernelGGL(dscores_states_kernel<E>, dim3(unsigned(n_dp + n_dql + ntb)), dim3(kThreads),
                       0, stream, a, int(n_dp), int(n_dql), ta, int(lin));
  }
  if (lin && pl.ng > 1) {
    CarryArgs<E> a{R(BR_DTT), R(BR_DCARRY), B, G, int(pl.ng), int(pl.gs), causal, int64_t(e) * s, 1};
    hipLaunchKernelGGL(carry_kernel<E>, dim3(unsigned(cdiv(pl.B * e * s / 8, 256))), dim3(256), 0,
                       stream, a);
  }
  if (lin) {
    XList<E> xl;
    xl.add(R(BR_DTT), R(BR_DTR), int(bp.slots), e, s);
    xl.launch(stream);
  }
  // ---- head gradients
  {
    DHeadsArgs<E> a{R(BR_DAR), R(BR_DAT), R(BR_KQT), R(BR_QQT), R(BR_VR), R(BR_DTR), Rf(BR_DQQ),
                    Rf(BR_DKQ), Rf(BR_DKL), nbg, G, c, s, e, causal};
    const int roles = lin ? 3 : 2;
    const int64_t per_role = pl.nbg * cdiv(c, bt) * cdiv(s, bt);
    hipLaunchKernelGGL(dheads_kernel<E>, dim3(unsigned(roles * per_role)), dim3(kThreads), 0, stream,
                       a, roles);
  }
  // ---- value gradients
  {
    DVArgs<E> a{R(BR_DVHT), R(BR_PT), R(BR_DTT), R(BR_KLR), R(BR_HR), R(BR_DHVR), R(BR_DHVT), nbg, G,
                c, s, e, causal, int(lin)};
    const int64_t nb = pl.nbg * cdiv(e, bt) * cdiv(c, bt);
    hipLaunchKernelGGL(dv_kernel<E>, dim3(unsigned(nb)), dim3(kThreads), 0, stream, a);
  }
  // ---- rotary transpose, dZ, dH_z, dγ/dβ partials
  {
    DZArgs<E> a{Rf(BR_DQQ), Rf(BR_DKQ), Rf(BR_DQL), Rf(BR_DKL), R(BR_HR), gamma, R(BR_DHZR),
                R(BR_DHZT), Rf(BR_GBPART), M, int(pl.n), c, e, s, int(lin), rope, log2_base};
    hipLaunchKernelGGL(dz_kernel<E>, dim3(unsigned(bp.nzb), unsigned(cdiv(s / 2, 256))), dim3(256), 0,
                       stream, a);
  }
  // ---- input gradient
  {
    DXArgs<E> a{reinterpret_cast<const T*>(W_u), reinterpret_cast<const T*>(W_v),
                reinterpret_cast<const T*>(W_z), R(BR_DHUR), R(BR_DHVR), R(BR_DHZR),
                reinterpret_cast<T*>(dX), M, d, e, s};
    const int64_t nb = cdiv(d, bt) * cdiv(M, bt);
    hipLaunchKernelGGL(dx_kernel<E>, dim3(unsigned(nb)), dim3(kThreads), 0, stream, a);
  }
  // ---- weight gradients
  float* wpart = Rf(BR_WPART);
  float* part[4];
  {
    int64_t o = 0;
    for (int i = 0; i < 4; ++i) {
      part[i] = wpart + o;
      o += bp.splits * bp.wcount[i];
    }
    WArgs<E> a{};
    const T* As[4] = {R(BR_XT), R(BR_XT), R(BR_XT), R(BR_YT)};
    const T* Bs[4] = {R(BR_DHUT), R(BR_DHVT), R(BR_DHZT), R(BR_DOT)};
    const int Fa[4] = {d, d, d, e};
    const int Fb[4] = {e, e, s, d};
    int total = 0;
    for (int i = 0; i < 4; ++i) {
      const int tm = int(cdiv(Fa[i], bt)), tn = int(cdiv(Fb[i], bt));
      a.job[i] = {As[i], Bs[i], part[i], Fa[i], Fb[i], tm, tn, total};
      total += int(bp.splits) * tm * tn;
    }
    a.njobs = 4;
    a.nbg = nbg;
    a.c = c;
    a.cps = int(bp.cps);
    a.splits = int(bp.splits);
    hipLaunchKernelGGL(wgrad_kernel<E>, dim3(unsigned(total)), dim3(kThreads), 0, stream, a, total);
  }
  // ---- reductions
  {
    RArgs<E> a{};
    void* outs[4] = {dW_u, dW_v, dW_z, dW_o};
    int64_t first = 0;
    for (int i = 0; i < 4; ++i) {
      a.job[i] = {part[i], reinterpret_cast<T*>(outs[i]), bp.wcount[i] / 4, first};
      first += bp.wcount[i] / 4;
    }
    a.njobs = 4;
    a.splits = int(bp.splits);
    hipLaunchKernelGGL(wreduce_kernel<E>, dim3(unsigned(cdiv(first, 256))), dim3(256), 0, stream, a,
                       first);
    hipLaunchKernelGGL(gbreduce_kernel, dim3(unsigned(cdiv(8 * s, 16))), dim3(1024), 0, stream,
                       Rf(BR_GBPART), int(bp.nzb), s, dgamma, dbeta);
  }
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

}  // namespace

extern "C" {

int flashgau_backward_workspace_size(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                                     int64_t chunk, int causal, flashgau_dtype dtype,
                                     size_t* out_bytes) {
  if (!out_bytes) return FLASHGAU_ERR_NULL_PTR;
  BPlan bp;
  const int rc = make_bplan(B, n, d, e, s, chunk, causal, dtype, &bp);
  if (rc != FLASHGAU_OK) return rc;
  *out_bytes = bp.total;
  return FLASHGAU_OK;
}

int flash_gau_backward(const void* X, const void* W_u, const void* W_v, const void* W_z,
                       const float* gamma, const float* beta, const void* W_o, const void* dO,
                       int64_t chunk, int causal, float rope_base, int64_t B, int64_t n, int64_t d,
                       int64_t e, int64_t s, flashgau_dtype dtype, void* dX, void* dW_u,
                       void* dW_v, void* dW_z, float* dgamma, float* dbeta, void* dW_o,
                       void* workspace, size_t workspace_bytes, void* hip_stream) {
  BPlan bp;
  const int rc = make_bplan(B, n, d, e, s, chunk, causal, dtype, &bp);
  if (rc != FLASHGAU_OK) return rc;
  if (!(rope_base >= 0.0f) || !std::isfinite(rope_base)) return FLASHGAU_ERR_BAD_SHAPE;
  if (rope_base > 0.0f && (s & 1)) return FLASHGAU_ERR_BAD_SHAPE;
  if (!dW_u || !dW_v || !dW_z || !dgamma || !dbeta || !dW_o) return FLASHGAU_ERR_NULL_PTR;
  const size_t es = size_t(bp.f.esz);
  const size_t nX = size_t(bp.f.M) * size_t(d) * es;
  const size_t nWu = size_t(d) * size_t(e) * es, nWz = size_t(d) * size_t(s) * es;
  const size_t nGB = size_t(4) * size_t(s) * sizeof(float);
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (misaligned(dW_u) || misaligned(dW_v) || misaligned(dW_z) || misaligned(dW_o) ||
      (reinterpret_cast<uintptr_t>(dgamma) & 3u) || (reinterpret_cast<uintptr_t>(dbeta) & 3u))
    return FLASHGAU_ERR_MISALIGNED;
  // the outputs must not overlap one another
  {
    void* outs[] = {dW_u, dW_v, dW_z, dW_o, dgamma, dbeta, dX};
    const size_t nout[] = {nWu, nWu, nWz, nWu, nGB, nGB, nX};
    const int cnt = bp.f.M > 0 ? 7 : 6;
    for (int i = 0; i < cnt; ++i)
      for (int j = i + 1; j < cnt; ++j)
        if (overlaps(outs[i], nout[i], outs[j], nout[j])) return FLASHGAU_ERR_ALIASING;
  }
  if (bp.f.M == 0) {
    // no tokens: every weight gradient is zero
    void* outs[] = {dW_u, dW_v, dW_z, dW_o, dgamma, dbeta};
    const size_t nout[] = {nWu, nWu, nWz, nWu, nGB, nGB};
    for (int i = 0; i < 6; ++i)
      hipLaunchKernelGGL(zero_kernel, dim3(unsigned(std::min<size_t>(1024, (nout[i] / 4 + 255) / 256))),
                         dim3(256), 0, stream, reinterpret_cast<uint32_t*>(outs[i]),
                         int64_t(nout[i] / 4));
    return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
  }
  if (!X || !W_u || !W_v || !W_z || !gamma || !beta || !W_o || !dO || !dX || !workspace)
    return FLASHGAU_ERR_NULL_PTR;
  if (misaligned(X) || misaligned(W_u) || misaligned(W_v) || misaligned(W_z) || misaligned(W_o) ||
      misaligned(dO) || misaligned(dX) || misaligned(workspace) ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return FLASHGAU_ERR_MISALIGNED;
  if (workspace_bytes < bp.total) return FLASHGAU_ERR_WORKSPACE;
  {
    const void* ins[] = {X, W_u, W_v, W_z, W_o, gamma, beta, dO};
    const size_t nin[] = {nX, nWu, nWu, nWz, nWu, nGB, nGB, nX};
    void* outs[] = {dW_u, dW_v, dW_z, dW_o, dgamma, dbeta, dX, workspace};
    const size_t nout[] = {nWu, nWu, nWz, nWu, nGB, nGB, nX, bp.total};
    for (int i = 0; i < 8; ++i)
      for (int j = 0; j < 8; ++j)
        if (overlaps(outs[j], nout[j], ins[i], nin[i])) return FLASHGAU_ERR_ALIASING;
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[j], nout[j], workspace, bp.total)) return FLASHGAU_ERR_ALIASING;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  const int cz = causal ? 1 : 0;
  if (dtype == FLASHGAU_BF16)
    return launch_backward<BF16>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, dO, cz, rope_base, dX, dW_u,
                                 dW_v, dW_z, dgamma, dbeta, dW_o, ws, stream);
  return launch_backward<F32>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, dO, cz, rope_base, dX, dW_u,
                              dW_v, dW_z, dgamma, dbeta, dW_o, ws, stream);
}

}  // extern "C"
