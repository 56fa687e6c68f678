// decode.hip — one causal decoding step of the FLASH layer for AMD Instinct MI355X (gfx950).
//
// The RNN form of causal linear attention (page "大模型训练之加速篇 -attention优化",
// blog.csdn.net, section 1.4: a running state updated token by token serves generation), joined to
// the causal "Mixed Chunk" layer of the page "FLASH: Possibly the Most Interesting Efficient
// Transformer Design Recently" (kexue.fm/archives/8934): token t of chunk g = t / c, position
// i = t mod c, reads
//   V̂_quad = Σ_{j<=i} relu(q_quad · k_quad_j / c)² v_j      over the keys of its own chunk
//   V̂_lin  = q_lin S / n,  S = Σ_{h<g} K_lin_hᵀ V_h           the state of the earlier chunks
//   o      = [u ⊙ (V̂_quad + V̂_lin)] W_o
// and after the chunk's last token the state takes in the chunk: S += K_lin_gᵀ V_g.
//
// One step for B sequences (all at position t) is three small launches, and a fourth after the
// last token of a chunk: with one token per sequence the work is reading the weights and the
// state once.
//   proj   h = x (W_u | W_v | W_z) for the B tokens: each workgroup owns 16 rows of the packed
//          (K-contiguous) weights and multiplies them with 16 token rows on the matrix cores, its
//          8 waves splitting K, operands fetched straight from global memory into fragments;
//          epilogue SiLU, the four heads, k_quad, k_lin and v written as row i of the chunk cache
//   attn   per sequence and 64 value columns: the weights relu(q·k_j / c)² for j <= i, then
//          Σ_j w_j v_j + q_lin S / n over the rows of the chunk cache and of the state, split over
//          64 row slots and reduced through LDS; y = u ⊙ (·)
//   out    o = y W_o, the same skinny matrix-core product as proj
//   fold   (after the last token of a chunk) S += K_linᵀ V of the chunk: the forward's tiled
//          matrix-core GEMM over the chunk's tokens, its epilogue adding into the fp32 state
// and at t = 0 a fill kernel clears S first.

#include <algorithm>
#include <cmath>

#include "kernels.h"

namespace {

// ------------------------------------------------------------------------------ skinny product
// With one token per sequence the projections are weight-streaming GEMVs: 16 weight rows times
// at most 16 token rows. kSplit waves share each 16-row slice, each taking 1/kSplit of K, so that
// enough bytes are in flight to stream the weights; their partial tiles are summed through LDS.
constexpr int kSplit = 8;
constexpr int kSkinnyThreads = 64 * kSplit;

// acc = A[16 rows] · Xr[16 rows]ᵀ over K elements [k0, k1) for one wave: lane l feeds row l % 16
// of both operands and the 16-byte chunk l / 16 of each K-step (the matrix-core fragment layout),
// so lane l ends with C[4 (l / 16) + r][l % 16], r = 0..3 (rows of A, then the Xr row). Four
// K-steps of loads are issued before their products.
template <class E>
__device__ __forceinline__ f32x4 skinny16(const Rows& a, const Rows& xr, int k0, int k1, int lane) {
  constexpr int kElems = 16 / E::kSize;  // elements per 16-byte chunk
  constexpr int kStep = 4 * kElems;      // K covered by one mma()
  const int lr = lane & 15, q = lane >> 4;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int kb = k0; kb < k1; kb += 4 * kStep) {
    u32x4 fa[4], fx[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = kb + u * kStep + q * kElems;
      const bool in = k < k1;
      fa[u] = load16(a, in ? uint32_t(lr) * a.ld + uint32_t(k) * E::kSize : kOutOfRange);
      fx[u] = load16(xr, in ? uint32_t(lr) * xr.ld + uint32_t(k) * E::kSize : kOutOfRange);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) mma(acc, fa[u], fx[u], E());
  }
  return acc;
}

// The whole workgroup's product for one 16-row slice: wave w takes its share of K (a multiple of
// the K-step, so chunks never straddle two waves), then the partial tiles are summed through LDS.
// Every lane of wave 0 returns the sum in its fragment position; other waves' results are unused.
template <class E>
__device__ __forceinline__ f32x4 skinny16_split(const Rows& a, const Rows& xr, int K, int wave,
                                                int lane, float* red) {
  constexpr int kStep = 4 * (16 / E::kSize);
  const int steps = (K + kStep - 1) / kStep;
  const int per = (steps + kSplit - 1) / kSplit;
  const int k0 = min(K, wave * per * kStep), k1 = min(K, (wave + 1) * per * kStep);
  const f32x4 acc = skinny16<E>(a, xr, k0, k1, lane);
#pragma unroll
  for (int r = 0; r < 4; ++r) red[(wave * 4 + r) * 64 + lane] = acc[r];
  __syncthreads();
  f32x4 sum = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kSplit; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) sum[r] += red[(w * 4 + r) * 64 + lane];
  }
  return sum;
}

// ------------------------------------------------------------------------------ proj
template <class E>
struct DecProjArgs {
  const typename E::T* x;      // [B, d]
  const typename E::T* WcatT;  // [2e+s, d]
  const float* gamma;          // [4, s]
  const float* beta;           // [4, s]
  typename E::T* U;            // [B, e]
  typename E::T* Vc;           // [B, c, e]
  typename E::T* Qq;           // [B, s]
  typename E::T* Kqc;          // [B, c, s]
  typename E::T* Ql;           // [B, s]
  typename E::T* Klc;          // [B, c, s]
  int B, d, e, s, c, i;
  int64_t t;         // position of the token
  int rope;          // rotate the four heads (rotary position embedding)
  double log2_base;  // log2 of the rotary base
};

// grid (ceil((2e+s) / 16), ceil(B / 16)), kSkinnyThreads threads: weight rows 16 x .. 16 x + 15.
template <class E>
__global__ __launch_bounds__(kSkinnyThreads) void dec_proj_kernel(DecProjArgs<E> p) {
  __shared__ float red[kSplit * 4 * 64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int ncols = 2 * p.e + p.s;
  const int col0 = blockIdx.x * 16;
  const int b0 = blockIdx.y * 16;
  const int64_t ld = int64_t(p.d) * E::kSize;
  const Rows a = make_rows(p.WcatT, col0, ld, min(16, ncols - col0));
  const Rows xr = make_rows(p.x, b0, ld, min(16, p.B - b0));
  const f32x4 acc = skinny16_split<E>(a, xr, p.d, wave, lane, red);
  if (wave != 0) return;

  const int b = b0 + (lane & 15);
  const int j = col0 + 4 * (lane >> 4);  // first of four consecutive output columns
  if (b >= p.B || j >= ncols) return;
  float y[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) y[r] = silu(acc[r]);
  // e and s are multiples of 8, so the four columns never straddle U, V and the heads
  if (j < p.e) {
    store4(p.U + int64_t(b) * p.e + j, y[0], y[1], y[2], y[3]);
  } else if (j < 2 * p.e) {
    store4(p.Vc + (int64_t(b) * p.c + p.i) * p.e + (j - p.e), y[0], y[1], y[2], y[3]);
  } else {
    const int jj = j - 2 * p.e;
    float h[4][4];  // [head][feature jj + r]
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) h[k][r] = fmaf(p.gamma[k * p.s + jj + r], y[r], p.beta[k * p.s + jj + r]);
    if (p.rope) {
      // jj % 4 == 0: the lane holds the rotary pairs (jj, jj+1) and (jj+2, jj+3) itself
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        float cs, sn;
        rope_angle(p.t, rope_theta(jj + r, p.s, p.log2_base), &cs, &sn);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = h[k][r], x1 = h[k][r + 1];
          h[k][r] = rope_apply(x0, x1, jj + r, cs, sn);
          h[k][r + 1] = rope_apply(x1, x0, jj + r + 1, cs, sn);
        }
      }
    }
    const int64_t row = int64_t(b) * p.s + jj;
    const int64_t crow = (int64_t(b) * p.c + p.i) * p.s + jj;
    store4(p.Qq + row, h[0][0], h[0][1], h[0][2], h[0][3]);
    store4(p.Kqc + crow, h[1][0], h[1][1], h[1][2], h[1][3]);
    store4(p.Ql + row, h[2][0], h[2][1], h[2][2], h[2][3]);
    store4(p.Klc + crow, h[3][0], h[3][1], h[3][2], h[3][3]);
  }
}

// ------------------------------------------------------------------------------ attn
template <class E>
struct DecAttnArgs {
  const typename E::T* Qq;   // [B, s]
  const typename E::T* Kqc;  // [B, c, s]
  const typename E::T* Ql;   // [B, s]
  const typename E::T* Vc;   // [B, c, e]
  const float* S;            // [B, s, e]
  const typename E::T* U;    // [B, e]
  typename E::T* Y;          // [B, e]
  int B, e, s, c, i;
  float inv_c, inv_n;
};

constexpr int kAttnCols = 64;    // value columns per workgroup (e / 64 x B workgroups)
constexpr int kAttnGroups = kAttnCols / 8;  // groups of 8 consecutive columns
constexpr int kAttnThreads = 512;
constexpr int kAttnSlots = kAttnThreads / kAttnGroups;  // row slots (64)
constexpr int kPreV = 2, kPreS = 2;  // cache and state rows per slot loaded before the key weights

// grid (ceil(e / 64), B), 512 threads, dynamic LDS (c + 2 s + 64·64) floats.
template <class E>
__global__ __launch_bounds__(kAttnThreads) void dec_attn_kernel(DecAttnArgs<E> p) {
  extern __shared__ float sh[];
  float* part = sh;                             // [kAttnSlots][kAttnCols] partial sums
  float* qq = part + kAttnSlots * kAttnCols;    // [s]
  float* ql = qq + p.s;                         // [s]
  float* w = ql + p.s;                          // [i + 1]
  const int tid = threadIdx.x;
  const int b = blockIdx.y;
  const int col0 = blockIdx.x * kAttnCols;
  // slot `sl` takes cache and state rows sl, sl + kAttnSlots, ...; group `cg` owns 8 consecutive
  // value columns. The first kPreV cache rows and kPreS state rows of the slot are loaded here,
  // before the key weights: they do not depend on them, so their latency overlaps that phase.
  const int cg = tid % kAttnGroups, sl = tid / kAttnGroups;
  const int col = col0 + cg * 8;
  const bool col_ok = col < p.e;  // e % 8 == 0: the 8 columns are all valid or all past the end
  const typename E::T* vb = p.Vc + int64_t(b) * p.c * p.e + col;
  const float* sb = p.S + int64_t(b) * p.s * p.e + col;
  float pv[kPreV][8], ps[kPreS][8];
#pragma unroll
  for (int r = 0; r < kPreV; ++r) {
    const int j = sl + r * kAttnSlots;
    if (col_ok && j <= p.i) {
      load8(vb + int64_t(j) * p.e, pv[r]);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) pv[r][m] = 0.f;
    }
  }
#pragma unroll
  for (int r = 0; r < kPreS; ++r) {
    const int k = sl + r * kAttnSlots;
    if (col_ok && k < p.s) {
      load8(sb + int64_t(k) * p.e, ps[r]);
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) ps[r][m] = 0.f;
    }
  }
  for (int k = tid; k < p.s; k += kAttnThreads) {
    qq[k] = to_f32(p.Qq[int64_t(b) * p.s + k]);
    ql[k] = to_f32(p.Ql[int64_t(b) * p.s + k]) * p.inv_n;
  }
  __syncthreads();
  // local weights w_j = relu(q·k_j / c)² of the keys 0..i of this chunk: four neighbouring lanes
  // per key, each summing every fourth 8-element chunk of the dot product (independent loads in
  // flight), combined by two lane exchanges that every lane executes
  const int nchunk = p.s / 8;
  for (int j0 = 0; j0 <= p.i; j0 += kAttnThreads / 4) {
    const int j = j0 + (tid >> 2), quarter = tid & 3;
    float dot = 0.f;
    if (j <= p.i) {
      const typename E::T* kr = p.Kqc + (int64_t(b) * p.c + j) * p.s;
#pragma unroll 4
      for (int ch = quarter; ch < nchunk; ch += 4) {
        float kv[8];
        load8(kr + ch * 8, kv);
#pragma unroll
        for (int m = 0; m < 8; ++m) dot = fmaf(qq[ch * 8 + m], kv[m], dot);
      }
    }
    dot += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dot), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    dot += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dot), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    if (j <= p.i && quarter == 0) {
      const float r = fmaxf(dot * p.inv_c, 0.f);
      w[j] = r * r;
    }
  }
  __syncthreads();

  // Σ_j w_j v_j over the cache rows and Σ_k (q_lin,k / n) S_k over the state rows: the prefetched
  // rows first, then the rest.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col_ok) {
#pragma unroll
    for (int r = 0; r < kPreV; ++r) {
      const int j = sl + r * kAttnSlots;
      const float wj = j <= p.i ? w[j] : 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(wj, pv[r][m], acc[m]);
    }
#pragma unroll
    for (int r = 0; r < kPreS; ++r) {
      const int k = sl + r * kAttnSlots;
      const float qk = k < p.s ? ql[k] : 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(qk, ps[r][m], acc[m]);
    }
#pragma unroll 4
    for (int j = sl + kPreV * kAttnSlots; j <= p.i; j += kAttnSlots) {
      float v[8];
      load8(vb + int64_t(j) * p.e, v);
      const float wj = w[j];
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(wj, v[m], acc[m]);
    }
#pragma unroll 4
    for (int k = sl + kPreS * kAttnSlots; k < p.s; k += kAttnSlots) {
      float v[8];
      load8(sb + int64_t(k) * p.e, v);
      const float qk = ql[k];
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(qk, v[m], acc[m]);
    }
  }
#pragma unroll
  for (int m = 0; m < 8; ++m) part[sl * kAttnCols + cg * 8 + m] = acc[m];
  __syncthreads();
  if (tid < kAttnCols && col0 + tid < p.e) {
    float sum = 0.f;
#pragma unroll 16
    for (int r = 0; r < kAttnSlots; ++r) sum += part[r * kAttnCols + tid];
    const int64_t o = int64_t(b) * p.e + col0 + tid;
    p.Y[o] = from_f32<E>(to_f32(p.U[o]) * sum);
  }
}

// ------------------------------------------------------------------------------ out
template <class E>
struct DecOutArgs {
  const typename E::T* WoT;  // [d, e]
  const typename E::T* Y;    // [B, e]
  typename E::T* O;          // [B, d]
  int B, d, e;
};

// grid (ceil(d / 16), ceil(B / 16)), kSkinnyThreads threads.
template <class E>
__global__ __launch_bounds__(kSkinnyThreads) void dec_out_kernel(DecOutArgs<E> p) {
  __shared__ float red[kSplit * 4 * 64];
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int col0 = blockIdx.x * 16;
  const int b0 = blockIdx.y * 16;
  const int64_t ld = int64_t(p.e) * E::kSize;
  const Rows a = make_rows(p.WoT, col0, ld, min(16, p.d - col0));
  const Rows yr = make_rows(p.Y, b0, ld, min(16, p.B - b0));
  const f32x4 acc = skinny16_split<E>(a, yr, p.e, wave, lane, red);
  if (wave != 0) return;
  const int b = b0 + (lane & 15);
  const int j = col0 + 4 * (lane >> 4);
  if (b < p.B && j < p.d) store4(p.O + int64_t(b) * p.d + j, acc[0], acc[1], acc[2], acc[3]);
}

// ------------------------------------------------------------------------------ fold
template <class E>
struct DecFoldArgs {
  const typename E::T* Klc;  // [B, c, s]
  const typename E::T* Vc;   // [B, c, e]
  float* S;                  // [B, s, e]
  int B, e, s, c;
};

// S_b += K_lin,gᵀ V_g on the matrix cores: one (state rows) x (value columns) tile of one sequence
// per workgroup, the contraction over the chunk's tokens reading the token-major cache rows as
// MN-major operands (K rows of s or e contiguous elements); the epilogue adds the tile to the fp32
// state in place.
template <class E> struct FoldShape;
template <> struct FoldShape<BF16> {
  static constexpr int BT = 128, WM = 2, WN = 4, NS = 2;  // an MN tile row is 256 bytes
};
template <> struct FoldShape<F32> {
  static constexpr int BT = 64, WM = 2, WN = 2, NS = 3;
};

// grid (ceil(s / BT), ceil(e / BT), B), 64 WM WN threads.
template <class E>
__global__ __launch_bounds__(64 * FoldShape<E>::WM * FoldShape<E>::WN) void dec_fold_kernel(
    DecFoldArgs<E> p) {
  using FS = FoldShape<E>;
  using G = TileGemm<E, FS::BT, FS::BT, FS::WM, FS::WN, FS::NS, false, 1, kLayoutMN, kLayoutMN>;
  __shared__ u32x4 lds[G::kLds];
  const int m0 = blockIdx.x * FS::BT;  // state row (K_lin dimension)
  const int n0 = blockIdx.y * FS::BT;  // value column
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int wm = wave / FS::WN, wn = wave % FS::WN;
  const Src a = make_src_mn(p.Klc, int64_t(b) * p.c, p.s, E::kSize, p.c, m0, p.s - m0);
  const Src v = make_src_mn(p.Vc, int64_t(b) * p.c, p.e, E::kSize, p.c, n0, p.e - n0);
  G g;
  g.zero();
  g.run(lds, (p.c + G::KS - 1) / G::KS,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = v;
          ka = kb = t * G::KS;
        },
        NoPre(), wave, wm, wn, lane);
  float* S = p.S + int64_t(b) * p.s * p.e;
  g.epilogue(wm, wn, lane, [&](int r, int cl, const f32x4& acc) {
    const int i = m0 + r, j = n0 + cl;  // rows i..i+3 of column j (s % 8 == 0)
    if (i >= p.s || j >= p.e) return;
#pragma unroll
    for (int k = 0; k < 4; ++k) S[int64_t(i + k) * p.e + j] += acc[k];
  });
}

// ------------------------------------------------------------------------------ clear
__global__ __launch_bounds__(256) void dec_clear_kernel(float* S, int64_t n4) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  for (int64_t k = blockIdx.x * int64_t(256) + threadIdx.x; k < n4; k += int64_t(gridDim.x) * 256)
    reinterpret_cast<f32x4*>(S)[k] = z;
}

// ------------------------------------------------------------------------------ host side
struct DecodePlan {
  int64_t B, d, e, s, c, esz, ncols;
  size_t off[FLASHGAU_DS_COUNT];
  size_t total;
};

int make_decode_plan(int64_t B, int64_t d, int64_t e, int64_t s, int64_t chunk,
                     flashgau_dtype dtype, DecodePlan* p) {
  if (dtype != FLASHGAU_F32 && dtype != FLASHGAU_BF16) return FLASHGAU_ERR_UNSUPPORTED;
  if (B < 0 || d < 1 || e < 1 || s < 1 || chunk < 1) return FLASHGAU_ERR_BAD_SHAPE;
  if (d % 8 || e % 8 || s % 8) return FLASHGAU_ERR_UNSUPPORTED;
  // the attention kernel keeps the chunk's weights and both query heads (chunk + 2 s floats, at
  // most 32 KB) in LDS next to its partial sums (at most 32 KB)
  static_assert(kAttnSlots * kAttnCols <= 8192, "at most 32 KB of partial sums");
  if (chunk + 2 * s > 8192) return FLASHGAU_ERR_UNSUPPORTED;
  p->B = B, p->d = d, p->e = e, p->s = s, p->c = chunk;
  p->esz = dtype == FLASHGAU_BF16 ? 2 : 4;
  p->ncols = 2 * e + s;
  int64_t bce, bcs, bse;
  if (!mul_ok(B * chunk, e, &bce) || !mul_ok(B * chunk, s, &bcs) || !mul_ok(B * s, e, &bse) ||
      B > kInt32Max / 16 || p->ncols > kInt32Max || B * chunk > kInt32Max || bce > kInt32Max ||
      bse > kInt32Max || d * p->esz > kInt32Max / 16 || e * p->esz > kInt32Max / 16)
    return FLASHGAU_ERR_BAD_SHAPE;
  const int64_t counts[FLASHGAU_DS_COUNT] = {bse, bcs, bcs, bce, B * e, B * s, B * s, B * e};
  size_t off = 0;
  for (int k = 0; k < FLASHGAU_DS_COUNT; ++k) {
    int64_t bytes;
    const int64_t esz = k == FLASHGAU_DS_S ? 4 : p->esz;  // the state is always fp32
    if (!mul_ok(counts[k], esz, &bytes)) return FLASHGAU_ERR_BAD_SHAPE;
    p->off[k] = off;
    const size_t padded = (size_t(bytes) + 255) & ~size_t(255);
    if (__builtin_add_overflow(off, padded, &off)) return FLASHGAU_ERR_BAD_SHAPE;
  }
  p->total = off;
  return FLASHGAU_OK;
}

template <class E>
int launch_decode(const DecodePlan& pl, const void* x, const char* packed, size_t wo_off,
                  const float* gamma, const float* beta, int64_t t, int64_t n, float rope_base,
                  void* o, char* st, hipStream_t stream) {
  using T = typename E::T;
  const int B = int(pl.B), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);
  const int i = int(t % pl.c);
  float* S = reinterpret_cast<float*>(st + pl.off[FLASHGAU_DS_S]);
  T* Kqc = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_KQ]);
  T* Klc = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_KL]);
  T* Vc = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_V]);
  T* U = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_U]);
  T* Qq = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_QQ]);
  T* Ql = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_QL]);
  T* Y = reinterpret_cast<T*>(st + pl.off[FLASHGAU_DS_Y]);
  const T* WcatT = reinterpret_cast<const T*>(packed);
  const T* WoT = reinterpret_cast<const T*>(packed + wo_off);

  if (t == 0) {
    const int64_t n4 = pl.B * pl.s * pl.e / 4;
    const int64_t nb = std::min<int64_t>(cdiv(n4, 256), 4096);
    hipLaunchKernelGGL(dec_clear_kernel, dim3(unsigned(nb)), dim3(256), 0, stream, S, n4);
  }
  {
    DecProjArgs<E> a{reinterpret_cast<const T*>(x), WcatT, gamma, beta, U, Vc, Qq, Kqc, Ql, Klc,
                     B, d, e, s, c, i, t, rope_base > 0.0f ? 1 : 0,
                     rope_base > 0.0f ? log2(double(rope_base)) : 0.0};
    hipLaunchKernelGGL(dec_proj_kernel<E>, dim3(unsigned(cdiv(pl.ncols, 16)), unsigned(cdiv(B, 16))),
                       dim3(kSkinnyThreads), 0, stream, a);
  }
  {
    DecAttnArgs<E> a{Qq, Kqc, Ql, Vc, S, U, Y, B, e, s, c, i, float(1.0 / double(c)),
                     float(1.0 / double(n))};
    const size_t lds = size_t(kAttnSlots * kAttnCols + 2 * s + c) * sizeof(float);
    hipLaunchKernelGGL(dec_attn_kernel<E>, dim3(unsigned(cdiv(e, kAttnCols)), unsigned(B)),
                       dim3(kAttnThreads), lds, stream, a);
  }
  {
    DecOutArgs<E> a{WoT, Y, reinterpret_cast<T*>(o), B, d, e};
    hipLaunchKernelGGL(dec_out_kernel<E>, dim3(unsigned(cdiv(d, 16)), unsigned(cdiv(B, 16))),
                       dim3(kSkinnyThreads), 0, stream, a);
  }
  if (i == c - 1) {
    DecFoldArgs<E> a{Klc, Vc, S, B, e, s, c};
    using FS = FoldShape<E>;
    hipLaunchKernelGGL(dec_fold_kernel<E>,
                       dim3(unsigned(cdiv(s, FS::BT)), unsigned(cdiv(e, FS::BT)), unsigned(B)),
                       dim3(64 * FS::WM * FS::WN), 0, stream, a);
  }
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

}  // namespace

extern "C" {

int flashgau_decode_state_size(int64_t B, int64_t d, int64_t e, int64_t s, int64_t chunk,
                               flashgau_dtype dtype, size_t* out_bytes) {
  if (!out_bytes) return FLASHGAU_ERR_NULL_PTR;
  DecodePlan pl;
  const int rc = make_decode_plan(B, d, e, s, chunk, dtype, &pl);
  if (rc != FLASHGAU_OK) return rc;
  *out_bytes = pl.total;
  return FLASHGAU_OK;
}

int flashgau_decode_state_offsets(int64_t B, int64_t d, int64_t e, int64_t s, int64_t chunk,
                                  flashgau_dtype dtype, size_t* out_offsets) {
  if (!out_offsets) return FLASHGAU_ERR_NULL_PTR;
  DecodePlan pl;
  const int rc = make_decode_plan(B, d, e, s, chunk, dtype, &pl);
  if (rc != FLASHGAU_OK) return rc;
  memcpy(out_offsets, pl.off, sizeof(pl.off));
  return FLASHGAU_OK;
}

int flash_gau_decode_step(const void* x, const void* packed, size_t packed_bytes,
                          const float* gamma, const float* beta, int64_t chunk, int64_t t,
                          int64_t n, float rope_base, int64_t B, int64_t d, int64_t e, int64_t s,
                          flashgau_dtype dtype, void* o, void* state, size_t state_bytes,
                          void* hip_stream) {
  DecodePlan pl;
  int rc = make_decode_plan(B, d, e, s, chunk, dtype, &pl);
  if (rc != FLASHGAU_OK) return rc;
  if (n < 1 || t < 0 || t >= n) return FLASHGAU_ERR_BAD_SHAPE;
  if (!(rope_base >= 0.0f) || !std::isfinite(rope_base)) return FLASHGAU_ERR_BAD_SHAPE;
  size_t wo_off = 0, packed_total = 0;
  rc = packed_plan(d, e, s, dtype, &wo_off, &packed_total);
  if (rc != FLASHGAU_OK) return rc;
  if (B == 0) return FLASHGAU_OK;
  if (!x || !packed || !gamma || !beta || !o || !state) return FLASHGAU_ERR_NULL_PTR;
  if (misaligned(x) || misaligned(packed) || misaligned(o) || misaligned(state) ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return FLASHGAU_ERR_MISALIGNED;
  if (packed_bytes < packed_total || state_bytes < pl.total) return FLASHGAU_ERR_WORKSPACE;
  const size_t nx = size_t(B * d * pl.esz), no = nx, ng = size_t(4 * s * 4);
  const void* ins[4] = {x, packed, gamma, beta};
  const size_t in_sz[4] = {nx, packed_total, ng, ng};
  for (int k = 0; k < 4; ++k)
    if (overlaps(o, no, ins[k], in_sz[k]) || overlaps(state, pl.total, ins[k], in_sz[k]))
      return FLASHGAU_ERR_ALIASING;
  if (overlaps(o, no, state, pl.total)) return FLASHGAU_ERR_ALIASING;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  char* st = reinterpret_cast<char*>(state);
  const char* pk = reinterpret_cast<const char*>(packed);
  return dtype == FLASHGAU_BF16
             ? launch_decode<BF16>(pl, x, pk, wo_off, gamma, beta, t, n, rope_base, o, st, stream)
             : launch_decode<F32>(pl, x, pk, wo_off, gamma, beta, t, n, rope_base, o, st, stream);
}

}  // extern "C"
