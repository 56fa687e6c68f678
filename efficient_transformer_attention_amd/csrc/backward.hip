// backward.hip — gradients of the FLASH layer for AMD Instinct MI355X (gfx950, CDNA4).
//
// The layer is the one of the forward (page "FLASH: Possibly the Most Interesting Efficient
// Transformer Design Recently", sections "Initial Power", "Weak Attention", "Mixed Chunk"); the
// page motivates the chunked form by its parallel training and prints no gradient, so the steps
// below are the chain rule of the forward's steps, in reverse order, for the loss Σ O ⊙ dO:
//
//   recompute  pack, proj (also storing the pre-activations), H_u = X W_u on the output
//              projection's GEMM, per-chunk scores P and the exclusive prefix states S_g / n (the
//              forward's own kernels)
//   mixb       per (chunk, value-column tile, token tile) two GEMMs into two accumulators:
//              V̂ᵀ = [V_gᵀ | S_gᵀ][P_g | Q_lin,g]ᵀ and dYᵀ = W_o dOᵀ; epilogue, with H_u = X W_u from
//              the projection: Y = U ⊙ V̂ (for dW_o), dV̂ = dY ⊙ U, dH_u = dY ⊙ V̂ ⊙ SiLU'(H_u)
//   dscores    per chunk dW = dV̂ Vᵀ and A = Q_quad K_quadᵀ again: dA = dW ⊙ 2 relu(A/c) / c
//              (masked); dQ_lin = dV̂ (S_g/n)ᵀ; and, in the same launch, the state gradients
//              dS_g = Q_lin,gᵀ dV̂_g / n summed over the LATER chunks (the forward's states and
//              carry kernels walking the chunks last to first)
//   dheads_dv  one launch: dQ_quad = dA K_quad, dK_quad = dAᵀ Q_quad, dK_lin = V dTᵀ, and
//              dVᵀ = [dV̂ᵀ | dTᵀ][Pᵀ | K_lin]ᵀ per chunk, times SiLU'(H_v)
//   dz         the rotary transpose, dZ = Σ γ_h dhead_h, dH_z, and partial sums for dγ, dβ
//   dx_wgrad   one launch: dX = dH_u W_uᵀ + dH_v W_vᵀ + dH_z W_zᵀ (the input weights as stored),
//              and dW = Xᵀ dH, dW_o = Yᵀ dO split over token ranges into fp32 partials
//   reduce     partial sums → dW_u, dW_v, dW_z, dW_o, dγ, dβ
//
// Every GEMM is the forward's TileGemm. A contraction over tokens (a chunk's, or all of them)
// reads its token-major operands as MN-major tiles (K rows of M-contiguous elements, fragments
// through the transposing LDS reads), so every intermediate is stored once, token-major, and
// nothing is transposed in memory. Tiles are 128 x 128 with 8 waves for bf16 and 64 x 64 with
// 4 waves for fp32 (one 256-byte column block per MN-major operand), except the input and weight
// gradients, which bf16 runs on 256 x 256 tiles (two column blocks).

#include <mutex>
#include <vector>

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

constexpr int KK = kLayoutK, MN = kLayoutMN;

template <class E, int AL = KK, int BL = KK>
using BGemm = TileGemm<E, BShapes<E>::BT, BShapes<E>::BT, BShapes<E>::WM, BShapes<E>::WN,
                       BShapes<E>::NS, false, 1, AL, BL>;

// The input and weight gradients are the longest contractions (over the 2e + s gate features, or
// over a token range): bf16 runs them on 256 x 256 tiles, 8 waves of 128 x 64 with a
// single-barrier two-stage ring, which read half the LDS fragment bytes per product that the
// 128 x 128 tiles' 64 x 32 wave tiles do. The fp32 partials of such a tile are staged in two
// passes (the whole wave tile would not fit the LDS tiles).
template <class E> struct XShapes;
template <> struct XShapes<BF16> {
  static constexpr int BT = 256, WM = 2, WN = 4, NS = 2, kPasses = 2;
  static constexpr bool SB = true;
};
template <> struct XShapes<F32> {
  static constexpr int BT = 64, WM = 2, WN = 2, NS = 3, kPasses = 1;
  static constexpr bool SB = false;
};
template <class E, int AL = KK, int BL = KK>
using XGemm = TileGemm<E, XShapes<E>::BT, XShapes<E>::BT, XShapes<E>::WM, XShapes<E>::WN,
                       XShapes<E>::NS, false, 1, AL, BL, XShapes<E>::SB>;

template <class E>
__device__ __forceinline__ int ksteps(int elems) {
  return (elems * E::kSize + kStageBytes - 1) / kStageBytes;
}

// K advance per tile of an operand: bytes along the row (K-major) or K rows (MN-major).
template <class G, bool IS_A>
constexpr int kadv() {
  return (IS_A ? G::kAL : G::kBL) == KK ? kStageBytes : G::KS;
}

// One tile of C = A Bᵀ over nk K-tiles from the offsets ka0, kb0 (bytes or rows, by layout),
// stored fp32 row-major at out (pitch ldo), rows < rows and columns < cols only.
template <class G, int PASSES = 1>
__device__ __forceinline__ void gemm_to_f32(u32x4* lds, const Src& a, int ka0, const Src& b, int kb0,
                                            int nk, float* out, int64_t ldo, int rows, int cols) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / G::kWN, wn = wave % G::kWN;
  G g;
  g.zero();
  g.run(lds, nk,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = b;
          ka = ka0 + t * kadv<G, true>();
          kb = kb0 + t * kadv<G, false>();
        },
        NoPre(), wave, wm, wn, lane);
  g.template stage_cols<float, PASSES>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, float* o) {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = v[k];
      },
      [&](int r, int cl, const u32x4& chunk) {
        if (r < rows && cl < cols) store16_stream(out + r * ldo + cl, chunk);
      });
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
  T* Yr;         // [M, e]
  T* dVhr;       // [M, e]
  T* dHur;       // [M, e]
  int d, nbg, G, c, e, s, causal, lin;
  int write_y;   // 0: Y is already in the workspace (the training forward wrote the same values)
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

  G gd;  // dYᵀ
  gd.zero();
  {
    const Src a = make_src(p.Wo, m0, p.d, E::kSize, p.e - m0, BT, p.d);
    const Src b = make_src(p.dO, tok0 + n0, p.d, E::kSize, p.c - n0, BT, p.d);
    gd.run(lds, ksteps<E>(p.d),
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

  // H_u of the tile (token rows, value columns) goes once into the LDS half that the output
  // staging leaves free; each of the three passes reads its four values from there.
  static_assert(2 * BT * BT * E::kSize <= G::kLds * 16, "H_u tile and staging exceed the LDS");
  char* const hub = reinterpret_cast<char*>(lds) + BT * BT * E::kSize;
  lds_tile_load<T, BT, BT, G::kThreads>(hub, p.Hu + (tok0 + n0) * p.e + m0, p.e, p.c - n0,
                                        p.e - m0);
  __syncthreads();
  auto load_hu = [&](int r, int cl, float* hu) { lds_tile_read4f<T, BT>(hub, cl, r, hu); };
  // what: 0 Y = U ⊙ V̂, 1 dV̂ = dY ⊙ U, 2 dH_u = dY ⊙ V̂ ⊙ SiLU'(H_u); all token-major
  T* const dst[3] = {p.Yr, p.dVhr, p.dHur};
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    if (w == 0 && !p.write_y) continue;
    g.template stage_rows<T>(
        lds, wave, wm, wn, lane,
        [&](int fi, int fj, int r, int cl, const f32x4& v, T* out) {
          float hu[4];
          load_hu(r, cl, hu);
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const float dy = gd.acc[fi][fj][k];
            const float x = w == 0 ? silu(hu[k]) * v[k]
                            : w == 1 ? dy * silu(hu[k])
                                     : dy * v[k] * silu_grad(hu[k]);
            out[k] = from_f32<E>(x);
          }
        },
        [&](int cl, int r, const u32x4& chunk) {
          const int j = m0 + r, i = n0 + cl;
          if (j < p.e && i < p.c) store16_stream(dst[w] + (tok0 + i) * p.e + j, chunk);
        });
  }
}

// ------------------------------------------------------------------------------ dscores
template <class E>
struct DScoresArgs {
  using T = typename E::T;
  const T* dVhr;  // [M, e]
  const T* Vt;    // [nbg, e, c]
  const T* Qq;    // [M, s]
  const T* Kq;    // [M, s]
  const T* St;    // [slots, e, s] (already / n)
  T* dAr;         // [nbg, c, c]: dA[i][j]
  float* dQl;     // [M, s]
  int nbg, G, c, s, e, causal;
  float inv_c;
};

// Tile (i-tile, j-tile) of one chunk: dW = dV̂ Vᵀ (over e; V read from V_gᵀ as an MN-major
// operand) and A = Q_quad K_quadᵀ (over s); dA = dW ⊙ 2 relu(A/c) / c, zero above the diagonal
// when causal. Causal launches only the tiles on or below the diagonal; the consumers read no other.
template <class E>
__device__ __forceinline__ void dp_block(const DScoresArgs<E>& p, u32x4* lds, int bid) {
  using GA = BGemm<E>;
  using GP = BGemm<E, KK, MN>;
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

  GA ga;
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
  GP gp;
  gp.zero();
  {
    const Src a = make_src(p.dVhr, tok0 + i0, p.e, E::kSize, p.c - i0, BT, p.e);
    const Src b = make_src_mn(p.Vt, int64_t(bg) * p.e, p.c, E::kSize, p.e, j0, p.c - j0);
    gp.run(lds, ksteps<E>(p.e),
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = a;
             sb = b;
             ka = t * kStageBytes;
             kb = t * GP::KS;
           },
           NoPre(), wave, wm, wn, lane);
  }
  gp.template stage_cols<T>(
      lds, wave, wm, wn, lane,
      [&](int fi, int fj, int r, int cl, const f32x4&, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int i = i0 + r + k, j = j0 + cl;
          const float x = fmaxf(ga.acc[fi][fj][k] * p.inv_c, 0.0f);
          out[k] = from_f32<E>((p.causal && j > i) ? 0.0f : gp.acc[fi][fj][k] * 2.0f * x * p.inv_c);
        }
      },
      [&](int r, int cl, const u32x4& chunk) {
        const int i = i0 + r, j = j0 + cl;
        if (i < p.c && j < p.c) store16_stream(p.dAr + (tok0 + i) * p.c + j, chunk);
      });
}

// dQ_lin = dV̂ (S_g/n)ᵀ per (chunk, token tile, feature tile); S/n read from its [e, s] layout as
// an MN-major operand.
template <class E>
__device__ __forceinline__ void dql_block(const DScoresArgs<E>& p, u32x4* lds, int bid) {
  constexpr int BT = BShapes<E>::BT;
  const int ntc = (p.c + BT - 1) / BT, nts = (p.s + BT - 1) / BT;
  const int lid = xcd_remap(bid, p.nbg * ntc * nts);
  const int bg = lid / (ntc * nts);
  const int rem = lid % (ntc * nts);
  const int i0 = (rem / nts) * BT, f0 = (rem % nts) * BT;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const int64_t row0 = int64_t(bg) * p.c + i0;
  const Src a = make_src(p.dVhr, row0, p.e, E::kSize, p.c - i0, BT, p.e);
  const Src b = make_src_mn(p.St, slot * p.e, p.s, E::kSize, p.e, f0, p.s - f0);
  gemm_to_f32<BGemm<E, KK, MN>>(lds, a, 0, b, 0, ksteps<E>(p.e), p.dQl + row0 * p.s + f0, p.s,
                                p.c - i0, p.s - f0);
}

// One launch, three roles by workgroup index: [0, n_dp) score-gradient tiles, [n_dp, n_dp +
// n_dql) dQ_lin tiles, then the state-gradient tiles (the forward's summaries walking the chunks
// last to first, reading Q_lin and dV̂ token-major: Q_lin,gᵀ dV̂_g / n summed over the later chunks).
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dscores_states_kernel(
    DScoresArgs<E> p, int n_dp, int n_dql, StatesArgs<E> tp, int states_on) {
  constexpr int BT = BShapes<E>::BT, WM = BShapes<E>::WM, WN = BShapes<E>::WN, NS = BShapes<E>::NS;
  __shared__ u32x4 lds[BGemm<E>::kLds];
  const int bid = blockIdx.x;
  if (bid < n_dp) {
    dp_block<E>(p, lds, bid);
  } else if (bid < n_dp + n_dql) {
    dql_block<E>(p, lds, bid - n_dp);
  } else if (states_on) {
    states_block<E, BT, BT, WM, WN, NS, MN>(tp, lds, bid - n_dp - n_dql);
  }
}

// ------------------------------------------------------------------------------ dheads
template <class E>
struct DHeadsArgs {
  using T = typename E::T;
  const T* dAr;  // [nbg, c, c]
  const T* Kq;   // [M, s]
  const T* Qq;   // [M, s]
  const T* Vt;   // [nbg, e, c]
  const T* dTt;  // [slots, e, s] (already / n)
  float* dQq;    // [M, s]
  float* dKq;    // [M, s]
  float* dKl;    // [M, s]
  int nbg, G, c, s, e, causal;
};

// Per (chunk, token tile, feature tile), one of three roles:
//   0: dQ_quad = dA K_quad over the keys (up to the tile's diagonal when causal); K_quad MN-major;
//   1: dK_quad = dAᵀ Q_quad over the queries (from the tile's diagonal); dA and Q_quad MN-major;
//   2: dK_lin = V dTᵀ over e; V from V_gᵀ and dT/n from its [e, s] layout, both MN-major.
template <class E>
__device__ __forceinline__ void dheads_block(const DHeadsArgs<E>& p, u32x4* lds, int role, int lid) {
  constexpr int BT = BShapes<E>::BT;
  const int ntc = (p.c + BT - 1) / BT, nts = (p.s + BT - 1) / BT;
  const int bg = lid / (ntc * nts);
  const int rem = lid % (ntc * nts);
  const int r0 = (rem / nts) * BT, f0 = (rem % nts) * BT;  // token tile of the chunk, feature tile
  const int64_t tok0 = int64_t(bg) * p.c;
  const int rows = p.c - r0, cols = p.s - f0;
  if (role == 0) {
    const int kend = p.causal ? min(p.c, r0 + BT) : p.c;
    const Src a = make_src(p.dAr, tok0 + r0, p.c, E::kSize, rows, BT, p.c);
    const Src b = make_src_mn(p.Kq, tok0, p.s, E::kSize, p.c, f0, cols);
    gemm_to_f32<BGemm<E, KK, MN>>(lds, a, 0, b, 0, ksteps<E>(kend), p.dQq + (tok0 + r0) * p.s + f0,
                                  p.s, rows, cols);
  } else if (role == 1) {
    const int kbeg = p.causal ? r0 : 0;
    const Src a = make_src_mn(p.dAr, tok0, p.c, E::kSize, p.c, r0, rows);
    const Src b = make_src_mn(p.Qq, tok0, p.s, E::kSize, p.c, f0, cols);
    gemm_to_f32<BGemm<E, MN, MN>>(lds, a, kbeg, b, kbeg, ksteps<E>(p.c - kbeg),
                                  p.dKq + (tok0 + r0) * p.s + f0, p.s, rows, cols);
  } else {
    const int64_t slot = p.causal ? bg : bg / p.G;
    const Src a = make_src_mn(p.Vt, int64_t(bg) * p.e, p.c, E::kSize, p.e, r0, rows);
    const Src b = make_src_mn(p.dTt, slot * p.e, p.s, E::kSize, p.e, f0, cols);
    gemm_to_f32<BGemm<E, MN, MN>>(lds, a, 0, b, 0, ksteps<E>(p.e), p.dKl + (tok0 + r0) * p.s + f0,
                                  p.s, rows, cols);
  }
}

// ------------------------------------------------------------------------------ dv
template <class E>
struct DVArgs {
  using T = typename E::T;
  const T* dVhr;  // [M, e]
  const T* P;     // [nbg, c, c]: P[i][j]
  const T* dTt;   // [slots, e, s] (already / n)
  const T* Klt;   // [nbg, s, c]
  const T* Hr;    // [M, e+s] pre-activations
  T* dHvr;        // [M, e]
  int nbg, G, c, s, e, causal, lin;
};

// Tile (value columns, keys j of a chunk): dVᵀ = dV̂ᵀ P over the queries i >= j (causal: from the
// tile's diagonal on; dV̂ and P MN-major), then + dTᵀ K_linᵀ over s (K_lin MN-major from its
// chunk-transposed copy), times SiLU'(H_v).
template <class E>
__device__ __forceinline__ void dv_block(const DVArgs<E>& p, u32x4* lds, int lid) {
  using G0 = BGemm<E, MN, MN>;
  using G1 = BGemm<E, KK, MN>;
  using T = typename E::T;
  constexpr int BT = BShapes<E>::BT, WN = BShapes<E>::WN;
  const int nte = (p.e + BT - 1) / BT, ntc = (p.c + BT - 1) / BT;
  const int bg = lid / (nte * ntc);
  const int rem = lid % (nte * ntc);
  const int nt = rem / nte, mt = rem % nte;
  const int m0 = mt * BT, n0 = nt * BT;  // m: value column, n: key inside the chunk
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;
  const int64_t tok0 = int64_t(bg) * p.c;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const int kbeg = p.causal ? n0 : 0;
  G0 g0;
  g0.zero();
  {
    const Src a = make_src_mn(p.dVhr, tok0, p.e, E::kSize, p.c, m0, p.e - m0);
    const Src b = make_src_mn(p.P, tok0, p.c, E::kSize, p.c, n0, p.c - n0);
    g0.run(lds, ksteps<E>(p.c - kbeg),
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = a;
             sb = b;
             ka = kb = kbeg + t * G0::KS;
           },
           NoPre(), wave, wm, wn, lane);
  }
  G1 g;
#pragma unroll
  for (int i = 0; i < G1::TM; ++i)
#pragma unroll
    for (int j = 0; j < G1::TN; ++j) g.acc[i][j] = g0.acc[i][j];
  if (p.lin) {
    const Src a = make_src(p.dTt, slot * p.e + m0, p.s, E::kSize, p.e - m0, BT, p.s);
    const Src b = make_src_mn(p.Klt, int64_t(bg) * p.s, p.c, E::kSize, p.s, n0, p.c - n0);
    g.run(lds, ksteps<E>(p.s),
          [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
            sa = a;
            sb = b;
            ka = t * kStageBytes;
            kb = t * G1::KS;
          },
          NoPre(), wave, wm, wn, lane);
  }
  // dH_v = dV ⊙ SiLU'(H_v), in place; the H_v tile (key rows, value columns) comes through the
  // LDS half that the output staging leaves free
  static_assert(2 * BT * BT * E::kSize <= G0::kLds * 16, "H_v tile and staging exceed the LDS");
  char* const hub = reinterpret_cast<char*>(lds) + BT * BT * E::kSize;
  const int ncols = p.e + p.s;
  lds_tile_load<T, BT, BT, G0::kThreads>(hub, p.Hr + (tok0 + n0) * ncols + m0, ncols, p.c - n0,
                                         p.e - m0);
  __syncthreads();
  const int lr = lane & 15, q = lane >> 4;
#pragma unroll
  for (int i = 0; i < G1::TM; ++i)
#pragma unroll
    for (int j = 0; j < G1::TN; ++j) {
      float h[4];  // value columns r.. of key cl (tile-local)
      lds_tile_read4f<T, BT>(hub, wn * G1::WTN + j * 16 + lr, wm * G1::WTM + i * 16 + q * 4, h);
#pragma unroll
      for (int k = 0; k < 4; ++k) g.acc[i][j][k] *= silu_grad(h[k]);
    }
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int j = m0 + r, key = n0 + cl;
        if (j < p.e && key < p.c) store16_stream(p.dHvr + (tok0 + key) * p.e + j, chunk);
      });
}

// One launch for the head and value gradients, which read only the score and state gradients:
// the long dK_lin tiles (K = e) first, then the value tiles, then the short dQ_quad and dK_quad
// tiles, so the short work fills in behind the long.
template <class E>
__global__ __launch_bounds__(BGemm<E>::kThreads) void dheads_dv_kernel(DHeadsArgs<E> h, DVArgs<E> v,
                                                                       int n_lin, int n_dv,
                                                                       int per_role) {
  __shared__ u32x4 lds[BGemm<E>::kLds];
  int bid = blockIdx.x;
  if (bid < n_lin) {
    dheads_block<E>(h, lds, 2, xcd_remap(bid, n_lin));
    return;
  }
  bid -= n_lin;
  if (bid < n_dv) {
    dv_block<E>(v, lds, xcd_remap(bid, n_dv));
    return;
  }
  bid -= n_dv;
  const int role = bid / per_role;
  if (role < 2) dheads_block<E>(h, lds, role, xcd_remap(bid - role * per_role, per_role));
}

// ------------------------------------------------------------------------------ dz
constexpr int kZRows = 32;  // token rows per dz workgroup

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
  float* gbpart;        // [nzb, 8, s]: rows 0..3 dγ, 4..7 dβ partial sums of workgroup row block
  int M, n, c, e, s, lin, rope;
  double log2_base;
};

// One thread per feature pair (2f, 2f+1) and group of rows; the rotary transpose turns a pair
// back by −m·θ.
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
    for (int row = int(blockIdx.x) * kZRows + rg; row < row_end; row += RG) {
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
      T* o = p.dHzr + int64_t(row) * p.s + f0;
      o[0] = from_f32<E>(dz0 * silu_grad(hz0));
      o[1] = from_f32<E>(dz1 * silu_grad(hz1));
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
__device__ __forceinline__ void dx_block(const DXArgs<E>& p, u32x4* lds, int lid) {
  using G = XGemm<E>;
  using T = typename E::T;
  constexpr int BT = XShapes<E>::BT, WN = XShapes<E>::WN;
  const int ntd = (p.d + BT - 1) / BT;
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
        if (k < p.d && i < p.M) store16_stream(p.dX + int64_t(i) * p.d + k, chunk);
      });
}

// ------------------------------------------------------------------------------ wgrad
// out[q] [Fa, Fb] = Σ over the tokens [q tps, (q+1) tps) of A[token] [Fa] ⊗ B[token] [Fb]: both
// operands token-major, read as MN-major tiles; fp32 partial per split q.
template <class E>
struct WJob {
  const typename E::T* A;  // [M, Fa]
  const typename E::T* B;  // [M, Fb]
  float* out;
  int Fa, Fb, tiles_m, tiles_n, first;
};
template <class E>
struct WArgs {
  WJob<E> job[4];
  int njobs, M, tps, splits;
};

template <class E>
__device__ __forceinline__ void wgrad_block(const WArgs<E>& p, u32x4* lds, int lid) {
  using G = XGemm<E, MN, MN>;
  constexpr int BT = XShapes<E>::BT;
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
  const int tbeg = q * p.tps;
  const int ntok = min(p.M, tbeg + p.tps) - tbeg;
  const Src a = make_src_mn(J.A, tbeg, J.Fa, E::kSize, ntok, m0, J.Fa - m0);
  const Src b = make_src_mn(J.B, tbeg, J.Fb, E::kSize, ntok, n0, J.Fb - n0);
  float* const out = J.out + int64_t(q) * J.Fa * J.Fb + int64_t(m0) * J.Fb + n0;
  gemm_to_f32<G, XShapes<E>::kPasses>(lds, a, 0, b, 0, ksteps<E>(ntok), out, J.Fb, J.Fa - m0,
                                      J.Fb - n0);
}

// One launch for the input and weight gradients, which read the same finished inputs: the
// weight-gradient tiles first, then the dX tiles.
template <class E>
__global__ __launch_bounds__(XGemm<E>::kThreads) void dx_wgrad_kernel(DXArgs<E> x, WArgs<E> w,
                                                                      int n_w, int n_dx) {
  static_assert(XGemm<E>::kLds == XGemm<E, MN, MN>::kLds, "one LDS size for both tile kinds");
  __shared__ u32x4 lds[XGemm<E>::kLds];
  const int bid = blockIdx.x;
  if (bid < n_w)
    wgrad_block<E>(w, lds, xcd_remap(bid, n_w));
  else
    dx_block<E>(x, lds, xcd_remap(bid - n_w, n_dx));
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

// The last launch of the backward: blocks [0, nw) sum the split-K partials of the weight
// gradients (four values per thread, the splits in order); blocks from nw on sum dγ, dβ [4, s]
// each from the dz partials [nzb, 8, s] (16 outputs per block, 16 lanes per output each summing
// every 16th partial, then a fixed-order sum of the 16). One launch instead of two: both read
// only finished partials.
template <class E>
__global__ __launch_bounds__(256) void reduce_kernel(RArgs<E> p, int64_t total4, int nw,
                                                     const float* gbpart, int nzb, int s,
                                                     float* dgamma, float* dbeta) {
  __shared__ float red[16][16 + 1];
  if (int(blockIdx.x) < nw) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= total4) return;
    RJob<E> J = p.job[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (i < p.njobs && idx >= p.job[i].first4) J = p.job[i];
    const int64_t i4 = idx - J.first4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < p.splits; ++q) {
      const f32x4 v = reinterpret_cast<const f32x4*>(J.part)[int64_t(q) * J.count4 + i4];
      acc[0] += v[0];
      acc[1] += v[1];
      acc[2] += v[2];
      acc[3] += v[3];
    }
    store4(J.out + i4 * 4, acc[0], acc[1], acc[2], acc[3]);
    return;
  }
  const int o = threadIdx.x & 15, l = threadIdx.x >> 4;
  const int j = (int(blockIdx.x) - nw) * 16 + o;  // output index in [0, 8 s)
  const int64_t stride = int64_t(8) * s;
  float v = 0.0f;
  if (j < 8 * s) {
    int b = l;
    for (; b + 48 < nzb; b += 64) {
      const float x0 = gbpart[int64_t(b) * stride + j], x1 = gbpart[int64_t(b + 16) * stride + j];
      const float x2 = gbpart[int64_t(b + 32) * stride + j], x3 = gbpart[int64_t(b + 48) * stride + j];
      v += (x0 + x1) + (x2 + x3);
    }
    for (; b < nzb; b += 16) v += gbpart[int64_t(b) * stride + j];
  }
  red[l][o] = v;
  __syncthreads();
  if (l == 0 && j < 8 * s) {
    for (int k = 1; k < 16; ++k) v += red[k][o];
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
  BR_HU, BR_HR, BR_YR, BR_DVHR, BR_DHUR, BR_DAR, BR_DTT, BR_DCARRY, BR_DQQ, BR_DKQ, BR_DQL, BR_DKL,
  BR_DHVR, BR_DHZR, BR_WPART, BR_GBPART, BR_COUNT
};

struct BPlan {
  Plan f;                 // the forward's regions come first in the workspace
  int64_t slots;          // state slots: chunks (causal) or sequences
  int64_t splits, tps;    // weight gradients: token-range splits, tokens per split
  int64_t wcount[4];      // elements of dW_u, dW_v, dW_z, dW_o
  int64_t nzb;            // dz row blocks
  int64_t bt;             // backward tile
  int64_t xbt;            // tile of the input and weight gradients
  size_t off[BR_COUNT];
  size_t total;
};

// Token-range splits of the weight gradients. The input/weight-gradient launch hands its tiles
// out in launch order (the weight-gradient tiles, split after split, then the dX tiles) to
// whichever slot frees first; bf16's 128 KB tiles hold one slot per CU. The host replays that
// greedy schedule for each candidate split count and keeps the one that finishes first once the
// fp32 partials are charged: every split writes one fp32 copy of all four weight gradients,
// which the reduction reads back.
//
// Greedy placement of k equal tiles of w stages on slots that free at times t: the tiles start at
// the k smallest of the times t_i + j w (j >= 0), so a search for the k-th smallest start places
// them all at once, whatever k is.
void place_equal_tiles(std::vector<int64_t>& t, int64_t k, int64_t w) {
  if (k <= 0) return;
  auto starts_below = [&](int64_t T) {
    int64_t c = 0;
    for (int64_t x : t)
      if (x < T) c += (T - x + w - 1) / w;
    return c;
  };
  int64_t lo = *std::min_element(t.begin(), t.end()), hi = lo + (k - 1) * w;
  while (lo < hi) {  // the k-th smallest start
    const int64_t mid = lo + (hi - lo) / 2;
    if (starts_below(mid + 1) >= k) hi = mid; else lo = mid + 1;
  }
  int64_t rest = k - starts_below(lo);  // tiles that start exactly at lo
  for (int64_t& x : t) {
    int64_t c = x < lo ? (lo - x + w - 1) / w : 0;
    if (rest > 0 && x <= lo && (lo - x) % w == 0) {
      ++c;
      --rest;
    }
    x += c * w;
  }
}

struct SplitModel {
  int64_t slots;        // workgroups resident at once over the 256 CUs
  double stage_us;      // one K-stage of one tile on one slot
  int64_t tile_extra;   // prologue and epilogue of a tile, in stages
  double hbm_bytes_us;  // sustained HBM bytes per microsecond for the partials
};

double schedule_us(const SplitModel& m, int64_t tiles_per_split, int64_t splits, int64_t tps,
                   int64_t M, int64_t ks, int64_t n_dx, int64_t dx_stages, int64_t wtot) {
  std::vector<int64_t> t(size_t(m.slots), 0);
  const int64_t last = M - (splits - 1) * tps;
  place_equal_tiles(t, (splits - 1) * tiles_per_split, tps / ks + m.tile_extra);
  place_equal_tiles(t, tiles_per_split, cdiv(last, ks) + m.tile_extra);
  place_equal_tiles(t, n_dx, dx_stages + m.tile_extra);
  const int64_t span = *std::max_element(t.begin(), t.end());
  return double(span) * m.stage_us + double(splits) * double(wtot) * 8.0 / m.hbm_bytes_us;
}

// Tokens per split for a shape (a multiple of the stage's ks tokens); the last few answers are
// kept, since the search takes up to about a millisecond and a training loop repeats its shapes.
int64_t pick_tps(int64_t M, int64_t d, int64_t e, int64_t s, flashgau_dtype dtype, int64_t xbt,
                 int64_t ks) {
  struct Entry { int64_t M, d, e, s, dtype, tps; };
  static std::mutex mu;
  static Entry cache[8];
  static int next = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (const Entry& c : cache)
      if (c.tps && c.M == M && c.d == d && c.e == e && c.s == s && c.dtype == dtype) return c.tps;
  }
  // bf16: one 256 x 256 tile per CU at about half the CU's share of 2.5 PFLOP/s; fp32: three
  // 64 x 64 tiles per CU sharing half its share of 157.3 TFLOP/s; partials at about 5 TB/s.
  const bool bf = dtype == FLASHGAU_BF16;
  const double stage_flops = 2.0 * double(xbt) * double(xbt) * double(ks);
  const double cu_flops_us = (bf ? 2.5e9 : 157.3e6) / 256 * 0.5;
  const int64_t per_cu = bf ? 1 : 3;
  const SplitModel m{256 * per_cu, stage_flops / (cu_flops_us / double(per_cu)), 3, 5.0e6};
  const int64_t tiles_per_split = 2 * cdiv(d, xbt) * cdiv(e, xbt) + cdiv(d, xbt) * cdiv(s, xbt) +
                                  cdiv(e, xbt) * cdiv(d, xbt);
  const int64_t wtot = 3 * d * e + d * s;
  const int64_t n_dx = cdiv(d, xbt) * cdiv(M, xbt);
  const int64_t dx_stages = 2 * cdiv(e, ks) + cdiv(s, ks);
  const int64_t max_splits = std::min<int64_t>(64, cdiv(M, ks));
  double best = 0.0;
  int64_t best_tps = 0;
  for (int64_t want = 1; want <= max_splits; ++want) {
    const int64_t tps = cdiv(cdiv(M, want), ks) * ks;
    if (cdiv(M, tps) != want) continue;  // the same ranges as a smaller count
    const double t = schedule_us(m, tiles_per_split, want, tps, M, ks, n_dx, dx_stages, wtot);
    if (best_tps == 0 || t < best) {
      best = t;
      best_tps = tps;
    }
  }
  std::lock_guard<std::mutex> lock(mu);
  cache[next] = Entry{M, d, e, s, int64_t(dtype), best_tps};
  next = (next + 1) % 8;
  return best_tps;
}

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
  bp->xbt = dtype == FLASHGAU_BF16 ? XShapes<BF16>::BT : XShapes<F32>::BT;
  const int64_t bt = bp->bt, xbt = bp->xbt;
  bp->slots = causal ? nbg : B;
  const int64_t tiles_per_split = 2 * cdiv(d, xbt) * cdiv(e, xbt) + cdiv(d, xbt) * cdiv(s, xbt) +
                                  cdiv(e, xbt) * cdiv(d, xbt);
  const int64_t ks = kStageBytes / f.esz;  // tokens per K-stage
  bp->tps = pick_tps(M, d, e, s, dtype, xbt, ks);
  bp->splits = cdiv(M, bp->tps);
  bp->nzb = cdiv(M, kZRows);
  const int64_t esz = f.esz;
  int64_t cnt[BR_COUNT], sz[BR_COUNT];
  for (int i = 0; i < BR_COUNT; ++i) sz[i] = esz;
  int64_t t0;
  if (!mul_ok(M, e, &cnt[BR_HU])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(M, e + s, &cnt[BR_HR])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_YR] = cnt[BR_DVHR] = cnt[BR_DHUR] = cnt[BR_DHVR] = cnt[BR_HU];
  if (!mul_ok(M, chunk, &cnt[BR_DAR])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(bp->slots, s, &t0) || !mul_ok(t0, e, &cnt[BR_DTT])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(B * f.ng, e, &t0) || !mul_ok(t0, s, &cnt[BR_DCARRY])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(M, s, &cnt[BR_DQQ])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[BR_DKQ] = cnt[BR_DQL] = cnt[BR_DKL] = cnt[BR_DHZR] = cnt[BR_DQQ];
  sz[BR_DQQ] = sz[BR_DKQ] = sz[BR_DQL] = sz[BR_DKL] = 4;
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
  // grid sizes, and the byte ranges the MN-major operands address (32-bit buffer descriptors)
  const int64_t ntc = cdiv(chunk, bt), nts = cdiv(s, bt), nte = cdiv(e, bt);
  const int64_t grids[] = {
      nbg * nte * ntc,                                                        // mixb
      nbg * ntc * ntc + nbg * ntc * nts + B * f.ng * cdiv(s, bt) * cdiv(e, bt),  // dscores_states
      3 * nbg * ntc * nts + nbg * nte * ntc,                                  // dheads + dv
      cdiv(d, xbt) * cdiv(M, xbt) + bp->splits * tiles_per_split,             // dx + wgrad
      cdiv(wtot / 4, 256) + cdiv(8 * s, 16),                                  // reduce
      bp->nzb * cdiv(s / 2, 256),                                             // dz
  };
  for (int64_t g : grids)
    if (g > kMaxBlocks) return FLASHGAU_ERR_BAD_SHAPE;
  const int64_t widest = std::max<int64_t>({d, e + s, chunk});
  if (bp->tps * widest * esz > int64_t(0xFFFFFFFF) || e * chunk * esz > int64_t(0xFFFFFFFF))
    return FLASHGAU_ERR_BAD_SHAPE;
  return FLASHGAU_OK;
}

// ------------------------------------------------------------------------------ launches
// The forward's intermediates as the backward reads them: pack, the projection over W_v | W_z
// (also storing the pre-activations H_v | H_z), with `gate` the gate's pre-activations H_u, scores
// and prefix states. `flash_gau_backward` runs this first; `flash_gau_forward_train` runs it
// without `gate` as part of a forward (its mix stage writes H_u) and leaves it in the workspace.
template <class E>
void launch_recompute(const BPlan& bp, const void* X, const void* W_u, const void* W_v,
                      const void* W_z, const float* gamma, const float* beta, const void* W_o,
                      int causal, float rope_base, char* ws, hipStream_t stream, bool gate) {
  using T = typename E::T;
  using S = Shapes<E>;
  const Plan& pl = bp.f;
  auto W = [&](int r) { return reinterpret_cast<T*>(ws + pl.off[r]); };
  auto R = [&](int r) { return reinterpret_cast<T*>(ws + bp.off[r]); };
  T *WcatT = W(FLASHGAU_WS_WCAT_T), *WoT = W(FLASHGAU_WS_WO_T), *Vt = W(FLASHGAU_WS_VT);
  T *Qq = W(FLASHGAU_WS_QQ), *Kq = W(FLASHGAU_WS_KQ), *Ql = W(FLASHGAU_WS_QL);
  T *Klt = W(FLASHGAU_WS_KLT), *P = W(FLASHGAU_WS_P), *St = W(FLASHGAU_WS_ST);
  T* Carry = W(FLASHGAU_WS_CARRY);
  const T* Xp = reinterpret_cast<const T*>(X);
  const int M = int(pl.M), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);
  const int nbg = int(pl.nbg), G = int(pl.G), B = int(pl.B);
  const bool lin = !(causal && pl.G == 1);
  const int rope = rope_base > 0.0f ? 1 : 0;
  const double log2_base = rope ? log2(double(rope_base)) : 0.0;
  const float inv_n = float(1.0 / double(pl.n));
  launch_pack<E>(W_u, W_v, W_z, W_o, d, e, s, WcatT, WoT, stream);
  {
    ProjArgs<E> a{Xp, WcatT + int64_t(e) * d, Vt, Qq, Kq, Ql, Klt, gamma, beta, M, d, e, s, c,
                  int(pl.n), rope, log2_base, R(BR_HR)};
    launch_proj<E, true>(a, stream);
  }
  if (gate) {
    // the gate's pre-activations H_u = X W_u, token-major: the output projection's GEMM (and its
    // large tiles) with W_uᵀ, the first e rows of the packed weights, in W_oᵀ's place and X in Y's
    OutArgs<E> g{WcatT, Xp, R(BR_HU), M, e, d};
    launch_out<E>(g, stream);
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
}

// A forward that keeps what the backward needs: the recompute stages, then the forward's mix
// (which also writes the gate's pre-activations H_u) and output projection.
template <class E>
int launch_train_forward(const BPlan& bp, const void* X, const void* W_u, const void* W_v,
                         const void* W_z, const float* gamma, const float* beta, const void* W_o,
                         int causal, float rope_base, void* O, char* ws, hipStream_t stream) {
  using T = typename E::T;
  const Plan& pl = bp.f;
  auto W = [&](int r) { return reinterpret_cast<T*>(ws + pl.off[r]); };
  auto R = [&](int r) { return reinterpret_cast<T*>(ws + bp.off[r]); };
  const int M = int(pl.M), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);
  const bool lin = !(causal && pl.G == 1);
  launch_recompute<E>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, causal, rope_base, ws, stream,
                      false);
  {
    MixArgs<E> a{W(FLASHGAU_WS_VT), W(FLASHGAU_WS_ST), W(FLASHGAU_WS_P), W(FLASHGAU_WS_QL),
                 reinterpret_cast<const T*>(X), W(FLASHGAU_WS_WCAT_T), W(FLASHGAU_WS_Y), d,
                 int(pl.nbg), int(pl.G), c, e, s, causal, int(lin), R(BR_HU)};
    launch_mix<E, true>(a, stream);
  }
  {
    OutArgs<E> a{W(FLASHGAU_WS_WO_T), W(FLASHGAU_WS_Y), reinterpret_cast<T*>(O), M, d, e};
    launch_out<E>(a, stream);
  }
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

template <class E>
int launch_backward(const BPlan& bp, const void* X, const void* W_u, const void* W_v,
                    const void* W_z, const float* gamma, const float* beta, const void* W_o,
                    const void* dO, int causal, float rope_base, void* dX, void* dW_u, void* dW_v,
                    void* dW_z, float* dgamma, float* dbeta, void* dW_o, char* ws,
                    hipStream_t stream, bool recompute) {
  using T = typename E::T;
  constexpr int kThreads = BGemm<E>::kThreads;
  const Plan& pl = bp.f;
  auto R = [&](int r) { return reinterpret_cast<T*>(ws + bp.off[r]); };
  auto Rf = [&](int r) { return reinterpret_cast<float*>(ws + bp.off[r]); };
  auto W = [&](int r) { return reinterpret_cast<T*>(ws + pl.off[r]); };
  T *Vt = W(FLASHGAU_WS_VT), *Qq = W(FLASHGAU_WS_QQ), *Kq = W(FLASHGAU_WS_KQ);
  T *Ql = W(FLASHGAU_WS_QL), *Klt = W(FLASHGAU_WS_KLT), *P = W(FLASHGAU_WS_P), *St = W(FLASHGAU_WS_ST);
  const T* Xp = reinterpret_cast<const T*>(X);
  const T* dOp = reinterpret_cast<const T*>(dO);
  const int M = int(pl.M), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);
  const int nbg = int(pl.nbg), G = int(pl.G), B = int(pl.B);
  const int bt = int(bp.bt), xbt = int(bp.xbt);
  const bool lin = !(causal && pl.G == 1);
  const int rope = rope_base > 0.0f ? 1 : 0;
  const double log2_base = rope ? log2(double(rope_base)) : 0.0;
  const float inv_n = float(1.0 / double(pl.n));

  if (recompute)
    launch_recompute<E>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, causal, rope_base, ws, stream,
                        true);

  // ---- gate, output projection and V̂
  {
    // Without the recompute, the training forward's mix stage has already written Y = U ⊙ V̂ to
    // the forward's Y buffer, bitwise what this stage would write (the same GEMM, the same order
    // over K, the same epilogue): the weight gradients read it there.
    MixBArgs<E> a{Vt, St, P, Ql, R(BR_HU), reinterpret_cast<const T*>(W_o), dOp, R(BR_YR),
                  R(BR_DVHR), R(BR_DHUR), d, nbg, G, c, e, s, causal, int(lin), recompute ? 1 : 0};
    const int64_t nb = pl.nbg * cdiv(e, bt) * cdiv(c, bt);
    hipLaunchKernelGGL(mixb_kernel<E>, dim3(unsigned(nb)), dim3(kThreads), 0, stream, a);
  }
  // ---- score gradients, dQ_lin, state gradients (token-major Q_lin and dV̂, chunks last to first)
  {
    DScoresArgs<E> a{R(BR_DVHR), Vt, Qq, Kq, St, R(BR_DAR), Rf(BR_DQL), nbg, G, c, s, e, causal,
                     1.0f / float(c)};
    const int64_t ntc = cdiv(c, bt), nts = cdiv(s, bt);
    const int64_t n_dp = pl.nbg * (causal ? ntc * (ntc + 1) / 2 : ntc * ntc);
    const int64_t n_dql = lin ? pl.nbg * ntc * nts : 0;
    StatesArgs<E> ta{Ql, R(BR_DVHR), R(BR_DTT), R(BR_DCARRY), B, G, s, e, c, causal, int(pl.ng),
                     int(pl.gs), inv_n, 1};
    const int64_t ntb = lin ? pl.B * pl.ng * cdiv(s, bt) * cdiv(e, bt) : 0;
    hipLaunchKernelGGL(dscores_states_kernel<E>, dim3(unsigned(n_dp + n_dql + ntb)), dim3(kThreads),
                       0, stream, a, int(n_dp), int(n_dql), ta, int(lin));
  }
  if (lin && pl.ng > 1) {
    CarryArgs<E> a{R(BR_DTT), R(BR_DCARRY), B, G, int(pl.ng), int(pl.gs), causal, int64_t(e) * s, 1};
    hipLaunchKernelGGL(carry_kernel<E>, dim3(unsigned(cdiv(pl.B * e * s / 8, 256))), dim3(256), 0,
                       stream, a);
  }
  // ---- head and value gradients
  {
    DHeadsArgs<E> h{R(BR_DAR), Kq, Qq, Vt, R(BR_DTT), Rf(BR_DQQ), Rf(BR_DKQ), Rf(BR_DKL), nbg, G, c,
                    s, e, causal};
    DVArgs<E> v{R(BR_DVHR), P, R(BR_DTT), Klt, R(BR_HR), R(BR_DHVR), nbg, G, c, s, e, causal,
                int(lin)};
    const int64_t per_role = pl.nbg * cdiv(c, bt) * cdiv(s, bt);
    const int64_t n_lin = lin ? per_role : 0;
    const int64_t n_dv = pl.nbg * cdiv(e, bt) * cdiv(c, bt);
    hipLaunchKernelGGL(dheads_dv_kernel<E>, dim3(unsigned(n_lin + n_dv + 2 * per_role)),
                       dim3(kThreads), 0, stream, h, v, int(n_lin), int(n_dv), int(per_role));
  }
  // ---- rotary transpose, dZ, dH_z, dγ/dβ partials
  {
    DZArgs<E> a{Rf(BR_DQQ), Rf(BR_DKQ), Rf(BR_DQL), Rf(BR_DKL), R(BR_HR), gamma, R(BR_DHZR),
                Rf(BR_GBPART), M, int(pl.n), c, e, s, int(lin), rope, log2_base};
    hipLaunchKernelGGL(dz_kernel<E>, dim3(unsigned(bp.nzb), unsigned(cdiv(s / 2, 256))), dim3(256), 0,
                       stream, a);
  }
  // ---- input and weight gradients
  float* wpart = Rf(BR_WPART);
  float* part[4];
  {
    int64_t o = 0;
    for (int i = 0; i < 4; ++i) {
      part[i] = wpart + o;
      o += bp.splits * bp.wcount[i];
    }
    WArgs<E> a{};
    const T* As[4] = {Xp, Xp, Xp, recompute ? R(BR_YR) : W(FLASHGAU_WS_Y)};
    const T* Bs[4] = {R(BR_DHUR), R(BR_DHVR), R(BR_DHZR), dOp};
    const int Fa[4] = {d, d, d, e};
    const int Fb[4] = {e, e, s, d};
    int total = 0;
    for (int i = 0; i < 4; ++i) {
      const int tm = int(cdiv(Fa[i], xbt)), tn = int(cdiv(Fb[i], xbt));
      a.job[i] = {As[i], Bs[i], part[i], Fa[i], Fb[i], tm, tn, total};
      total += int(bp.splits) * tm * tn;
    }
    a.njobs = 4;
    a.M = M;
    a.tps = int(bp.tps);
    a.splits = int(bp.splits);
    DXArgs<E> x{reinterpret_cast<const T*>(W_u), reinterpret_cast<const T*>(W_v),
                reinterpret_cast<const T*>(W_z), R(BR_DHUR), R(BR_DHVR), R(BR_DHZR),
                reinterpret_cast<T*>(dX), M, d, e, s};
    const int64_t n_dx = cdiv(d, xbt) * cdiv(M, xbt);
    hipLaunchKernelGGL(dx_wgrad_kernel<E>, dim3(unsigned(total + n_dx)), dim3(XGemm<E>::kThreads), 0, stream,
                       x, a, total, int(n_dx));
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
    const int64_t nw = cdiv(first, 256);
    hipLaunchKernelGGL(reduce_kernel<E>, dim3(unsigned(nw + cdiv(8 * s, 16))), dim3(256), 0, stream,
                       a, first, int(nw), Rf(BR_GBPART), int(bp.nzb), s, dgamma, dbeta);
  }
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

// Host-side checks shared by the entry points that take the backward workspace: outs[i] holds
// nout[i] bytes (0: not used by this call) and must be aligned to amask[i] + 1 bytes.
int check_call(const BPlan& bp, const void* X, const void* W_u, const void* W_v, const void* W_z,
               const float* gamma, const float* beta, const void* W_o, const void* dO,
               float rope_base, void* const* outs, const size_t* nout, const uint32_t* amask,
               int nouts, void* workspace, size_t workspace_bytes) {
  if (!(rope_base >= 0.0f) || !std::isfinite(rope_base)) return FLASHGAU_ERR_BAD_SHAPE;
  for (int i = 0; i < nouts; ++i)
    if (nout[i] && !outs[i]) return FLASHGAU_ERR_NULL_PTR;
  for (int i = 0; i < nouts; ++i)
    if (nout[i] && (reinterpret_cast<uintptr_t>(outs[i]) & amask[i])) return FLASHGAU_ERR_MISALIGNED;
  for (int i = 0; i < nouts; ++i)
    for (int j = i + 1; j < nouts; ++j)
      if (overlaps(outs[i], nout[i], outs[j], nout[j])) return FLASHGAU_ERR_ALIASING;
  if (bp.f.M == 0) return FLASHGAU_OK;
  if (!X || !W_u || !W_v || !W_z || !gamma || !beta || !W_o || !workspace) return FLASHGAU_ERR_NULL_PTR;
  if (misaligned(X) || misaligned(W_u) || misaligned(W_v) || misaligned(W_z) || misaligned(W_o) ||
      (dO && misaligned(dO)) || misaligned(workspace) ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return FLASHGAU_ERR_MISALIGNED;
  if (workspace_bytes < bp.total) return FLASHGAU_ERR_WORKSPACE;
  const size_t es = size_t(bp.f.esz);
  const size_t nX = size_t(bp.f.M) * size_t(bp.f.d) * es;
  const size_t nWu = size_t(bp.f.d) * size_t(bp.f.e) * es, nWz = size_t(bp.f.d) * size_t(bp.f.s) * es;
  const size_t nGB = size_t(4) * size_t(bp.f.s) * sizeof(float);
  const void* ins[] = {X, W_u, W_v, W_z, W_o, gamma, beta, dO};
  const size_t nin[] = {nX, nWu, nWu, nWz, nWu, nGB, nGB, dO ? nX : 0};
  for (int i = 0; i < 8; ++i) {
    for (int j = 0; j < nouts; ++j)
      if (overlaps(outs[j], nout[j], ins[i], nin[i])) return FLASHGAU_ERR_ALIASING;
    if (overlaps(workspace, bp.total, ins[i], nin[i])) return FLASHGAU_ERR_ALIASING;
  }
  for (int j = 0; j < nouts; ++j)
    if (overlaps(outs[j], nout[j], workspace, bp.total)) return FLASHGAU_ERR_ALIASING;
  return FLASHGAU_OK;
}

int backward_impl(const void* X, const void* W_u, const void* W_v, const void* W_z,
                  const float* gamma, const float* beta, const void* W_o, const void* dO,
                  int64_t chunk, int causal, float rope_base, int64_t B, int64_t n, int64_t d,
                  int64_t e, int64_t s, flashgau_dtype dtype, void* dX, void* dW_u, void* dW_v,
                  void* dW_z, float* dgamma, float* dbeta, void* dW_o, void* workspace,
                  size_t workspace_bytes, void* hip_stream, bool recompute) {
  BPlan bp;
  const int rc = make_bplan(B, n, d, e, s, chunk, causal, dtype, &bp);
  if (rc != FLASHGAU_OK) return rc;
  if (rope_base > 0.0f && (s & 1)) return FLASHGAU_ERR_BAD_SHAPE;
  const size_t es = size_t(bp.f.esz);
  const size_t nX = size_t(bp.f.M) * size_t(d) * es;
  const size_t nWu = size_t(d) * size_t(e) * es, nWz = size_t(d) * size_t(s) * es;
  const size_t nGB = size_t(4) * size_t(s) * sizeof(float);
  void* outs[] = {dW_u, dW_v, dW_z, dW_o, dgamma, dbeta, dX};
  const size_t nout[] = {nWu, nWu, nWz, nWu, nGB, nGB, nX};
  const uint32_t amask[] = {15u, 15u, 15u, 15u, 3u, 3u, 15u};
  if (bp.f.M > 0 && !dO) return FLASHGAU_ERR_NULL_PTR;
  const int vc = check_call(bp, X, W_u, W_v, W_z, gamma, beta, W_o, dO, rope_base, outs, nout,
                            amask, 7, workspace, workspace_bytes);
  if (vc != FLASHGAU_OK) return vc;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  if (bp.f.M == 0) {
    // no tokens: every weight gradient is zero
    for (int i = 0; i < 6; ++i)
      hipLaunchKernelGGL(zero_kernel, dim3(unsigned(std::min<size_t>(1024, (nout[i] / 4 + 255) / 256))),
                         dim3(256), 0, stream, reinterpret_cast<uint32_t*>(outs[i]),
                         int64_t(nout[i] / 4));
    return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  const int cz = causal ? 1 : 0;
  if (dtype == FLASHGAU_BF16)
    return launch_backward<BF16>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, dO, cz, rope_base, dX, dW_u,
                                 dW_v, dW_z, dgamma, dbeta, dW_o, ws, stream, recompute);
  return launch_backward<F32>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, dO, cz, rope_base, dX, dW_u,
                              dW_v, dW_z, dgamma, dbeta, dW_o, ws, stream, recompute);
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
  return backward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal, rope_base, B, n, d, e,
                       s, dtype, dX, dW_u, dW_v, dW_z, dgamma, dbeta, dW_o, workspace,
                       workspace_bytes, hip_stream, true);
}

int flash_gau_backward_saved(const void* X, const void* W_u, const void* W_v, const void* W_z,
                             const float* gamma, const float* beta, const void* W_o,
                             const void* dO, int64_t chunk, int causal, float rope_base, int64_t B,
                             int64_t n, int64_t d, int64_t e, int64_t s, flashgau_dtype dtype,
                             void* dX, void* dW_u, void* dW_v, void* dW_z, float* dgamma,
                             float* dbeta, void* dW_o, void* workspace, size_t workspace_bytes,
                             void* hip_stream) {
  return backward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, dO, chunk, causal, rope_base, B, n, d, e,
                       s, dtype, dX, dW_u, dW_v, dW_z, dgamma, dbeta, dW_o, workspace,
                       workspace_bytes, hip_stream, false);
}

int flash_gau_forward_train(const void* X, const void* W_u, const void* W_v, const void* W_z,
                            const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                            int causal, float rope_base, int64_t B, int64_t n, int64_t d, int64_t e,
                            int64_t s, flashgau_dtype dtype, void* O, void* workspace,
                            size_t workspace_bytes, void* hip_stream) {
  BPlan bp;
  const int rc = make_bplan(B, n, d, e, s, chunk, causal, dtype, &bp);
  if (rc != FLASHGAU_OK) return rc;
  if (rope_base > 0.0f && (s & 1)) return FLASHGAU_ERR_BAD_SHAPE;
  if (bp.f.M == 0) return FLASHGAU_OK;
  void* outs[] = {O};
  const size_t nout[] = {size_t(bp.f.M) * size_t(d) * size_t(bp.f.esz)};
  const uint32_t amask[] = {15u};
  const int vc = check_call(bp, X, W_u, W_v, W_z, gamma, beta, W_o, nullptr, rope_base, outs, nout,
                            amask, 1, workspace, workspace_bytes);
  if (vc != FLASHGAU_OK) return vc;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  char* ws = reinterpret_cast<char*>(workspace);
  const int cz = causal ? 1 : 0;
  if (dtype == FLASHGAU_BF16)
    return launch_train_forward<BF16>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, cz, rope_base, O, ws,
                                      stream);
  return launch_train_forward<F32>(bp, X, W_u, W_v, W_z, gamma, beta, W_o, cz, rope_base, O, ws,
                                   stream);
}

}  // extern "C"
