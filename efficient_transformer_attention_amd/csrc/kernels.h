// kernels.h — the GEMM core, the forward kernels and their host-side plan, shared by the
// forward (flashgau.hip), the backward pass (backward.hip) and the decoder's state fold
// (decode.hip). Everything here lives in an anonymous namespace: each translation unit
// instantiates what it launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#include "flashgau.h"
#include "common.h"

namespace {


// Block-level tiled GEMM C[BM x BN] += A[BM x K] · B[BN x K]ᵀ (operand layouts below).
// WM x WN waves; each wave owns a (BM/WM) x (BN/WN) block of 16x16 accumulator fragments.
// Operand tiles travel from global memory straight into a ring of NS LDS stages (no staging
// registers): with NS = 3 the loads of tile t+2 fly while tile t is multiplied, one barrier per
// tile; with NS = 2 (tiles too large for three stages) the loads of tile t+2 are issued after
// tile t has been consumed, two barriers per tile, or, with SB (single barrier), the loads of
// tile t+1 are issued right after the barrier that opens tile t (the stage they fill held tile
// t-1, which every wave finished before that barrier), one barrier per tile. PRIO raises the
// wave priority while it issues matrix instructions; iglp_opt(1) asks the scheduler to
// interleave the LDS reads with them.
//
// Operand layouts (AL for A, BL for B): kLayoutK (the default) stores each of the tile's rows with
// its K elements contiguous; kLayoutMN stores the operand as K rows of M-contiguous elements (a
// token-major tensor read with K = tokens, say). An MN tile is one or more 256-byte column blocks,
// each KS K-rows of 256 bytes, stored one after the other; it travels into LDS as straight 1 KB
// copies whose source chunks are permuted (below), and
// its fragments are read with the transposing LDS reads of CDNA4 (ds_read_b64_tr_b16: in every
// 16-lane group, lane i's k-th element comes from lane i/4 + 4k at column offset i % 4), four
// 4-byte reads per fragment for fp32.
constexpr int kLayoutK = 0, kLayoutMN = 1;

template <class E, int BM, int BN, int WM, int WN, int NS = 3, bool PRIO = false, int IGLP = 1,
          int AL = kLayoutK, int BL = kLayoutK, bool SB = false>
struct TileGemm {
  static constexpr int kThreads = 64 * WM * WN;
  static constexpr int kWaves = WM * WN;
  static constexpr int WTM = BM / WM;
  static constexpr int WTN = BN / WN;
  static constexpr int TM = WTM / 16;
  static constexpr int TN = WTN / 16;
  static constexpr int kStage = (BM + BN) * kRowChunks;  // u32x4 elements per stage
  static constexpr int kLds = NS * kStage;
  static constexpr int IPW = (BM + BN) / 8 / kWaves;     // 8-row copies per wave and stage
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be a multiple of 16");
  static_assert((BM + BN) % (8 * kWaves) == 0, "tile rows must spread evenly over the waves");
  static_assert(NS == 2 || NS == 3, "two or three LDS stages");
  static_assert(BM % 8 == 0, "A rows end on an 8-row boundary");
  static constexpr int KS = kStageBytes / E::kSize;  // K elements per stage
  static constexpr int kWM = WM, kWN = WN, kAL = AL, kBL = BL;
  static_assert(AL == kLayoutK || (BM * E::kSize) % 256 == 0, "an MN-major A tile is 256-byte blocks");
  static_assert(BL == kLayoutK || (BN * E::kSize) % 256 == 0, "an MN-major B tile is 256-byte blocks");
  static constexpr int kMNSlabs = KS / 4;               // 1 KB slabs per 256-byte block of an MN tile
  static constexpr int kMNBlk = 256 / (16 * E::kSize);  // 16-element fragment blocks per 256 bytes

  // Chunk swizzle of an MN tile's K row p (even, so the two chunks of a 16-element fragment row
  // stay adjacent): the 8 K rows one transposing read serves per half-wave (p = 8g + r, r < 4,
  // g < 2) land in 8 distinct 32-byte bank windows.
  __device__ __forceinline__ static int mn_swizzle(int p) {
    return 2 * ((p & 3) | (((p >> 3) & 1) << 2));
  }

  f32x4 acc[TM][TN];

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Copies K-tile (a at ka, b at kb) into LDS stage `stage`. Each copy instruction fills one 1 KB
  // slab of the stage (A's slabs first, then B's). K-major operand: ka is the byte offset along K;
  // slab s holds rows [8s, 8s+8), lane l fetches row + l/8, logical chunk (l % 8) ^ (l / 8), which
  // lands at physical chunk l % 8: the XOR-swizzled layout. MN-major operand: ka is the first K
  // row; slab s fills column block s / kMNSlabs with its K rows [4r, 4r+4), r = s % kMNSlabs: lane
  // l fetches K row 4r + l/16, logical chunk (l % 16) ^ mn_swizzle(row) of the block, landing at
  // physical chunk l % 16; src.kbytes bounds the valid M bytes of a row, and rows past the
  // descriptor's range read as zeros.
  __device__ __forceinline__ static void issue(u32x4* lds, int stage, const Src& a, int ka,
                                               const Src& b, int kb, int wave, int lane) {
    const uint32_t base = uint32_t(reinterpret_cast<uintptr_t>(lds)) + uint32_t(stage * kStage) * 16;
    const int lchunk = (lane & 7) ^ (lane >> 3);
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      const int rg = wave * IPW + j;  // wave-uniform
      const bool is_a = rg * 8 < BM;
      const Src& src = is_a ? a : b;
      const int slab = is_a ? rg : rg - BM / 8;
      uint32_t voff;
      if ((is_a ? AL : BL) == kLayoutMN) {
        const int row = (slab % kMNSlabs) * 4 + (lane >> 4);
        const int col = (slab / kMNSlabs) * 256 + ((lane & 15) ^ mn_swizzle(row)) * 16;
        voff = col < src.kbytes ? uint32_t((is_a ? ka : kb) + row) * src.ld + uint32_t(col) : kOutOfRange;
      } else {
        const int row = slab * 8 + (lane >> 3);
        const int koff = (is_a ? ka : kb) + lchunk * 16;
        voff = koff < src.kbytes ? uint32_t(row) * src.ld + uint32_t(koff) : kOutOfRange;
      }
      lds_dma16(src.rsrc, voff, base + uint32_t(rg) * 1024u);
    }
  }

  // The lane's 16-byte fragment of rows [16 blk, 16 blk + 16) of an operand region R (K-major or
  // MN-major), sub-step ks of the stage: row lane % 16, K elements of lane group lane / 16.
  template <int L>
  __device__ __forceinline__ static u32x4 frag(const u32x4* R, int blk, int ks, int lane) {
    const int lr = lane & 15, q = lane >> 4;
    if constexpr (L == kLayoutK) {
      return R[(blk * 16 + lr) * kRowChunks + ((ks * 4 + q) ^ (lr & 7))];
    } else if constexpr (sizeof(typename E::T) == 2) {
      // K rows 32 ks + 8 q + lr/4 (+4), 8 bytes at column 16 blk + 4 (lr % 4)
      typedef short v4i16 __attribute__((ext_vector_type(4)));
      const char* base = reinterpret_cast<const char*>(R) + (blk / kMNBlk) * (KS * 256);
      const int cb = (blk % kMNBlk) * 32 + 8 * (lr & 3);  // byte within the block's K row
      const int p0 = 32 * ks + 8 * q + (lr >> 2);
      const int p1 = p0 + 4;
      const char* a0 = base + p0 * 256 + ((((cb >> 4) ^ mn_swizzle(p0)) << 4) | (cb & 15));
      const char* a1 = base + p1 * 256 + ((((cb >> 4) ^ mn_swizzle(p1)) << 4) | (cb & 15));
      const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(a0));
      const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16*)(a1));
      const u32x2 w0 = __builtin_bit_cast(u32x2, x0), w1 = __builtin_bit_cast(u32x2, x1);
      return u32x4{w0[0], w0[1], w1[0], w1[1]};
    } else {
      // fp32: the four K rows 16 ks + 4 q + c of column 16 blk + lr
      const char* base = reinterpret_cast<const char*>(R) + (blk / kMNBlk) * (KS * 256);
      const int cb = (blk % kMNBlk) * 64 + 4 * lr;
      u32x4 r;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int p = 16 * ks + 4 * q + c;
        r[c] = *reinterpret_cast<const uint32_t*>(base + p * 256 +
                                                  ((((cb >> 4) ^ mn_swizzle(p)) << 4) | (cb & 15)));
      }
      return r;
    }
  }

  template <class Tiles>
  __device__ __forceinline__ static void issue_tile(u32x4* lds, Tiles& tiles, int t, int wave,
                                                    int lane) {
    Src a, b;
    int ka, kb;
    tiles(t, a, ka, b, kb);
    issue(lds, t % NS, a, ka, b, kb, wave, lane);
  }

  __device__ __forceinline__ void compute(const u32x4* stage, int wm, int wn, int lane) {
    const u32x4* As = stage;
    const u32x4* Bs = stage + BM * kRowChunks;
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    if constexpr (IGLP >= 0) __builtin_amdgcn_iglp_opt(IGLP);
#pragma unroll
    for (int ks = 0; ks < kRowChunks / 4; ++ks) {
      u32x4 a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = frag<AL>(As, wm * TM + i, ks, lane);
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = frag<BL>(Bs, wn * TN + j, ks, lane);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) mma(acc[i][j], a[i], b[j], E());
    }
    if (PRIO) __builtin_amdgcn_s_setprio(0);
  }

  // Runs K-tiles 0..nt-1. tiles(t, a, ka, b, kb) names the operands and byte offsets of tile t;
  // pre(t) runs right before tile t is multiplied (it may read the accumulators). Returns with
  // every copy complete and every wave past a final barrier, so LDS may be reused.
  template <class Tiles, class Pre>
  __device__ __forceinline__ void run(u32x4* lds, int nt, Tiles&& tiles, Pre&& pre, int wave,
                                      int wm, int wn, int lane) {
    run(lds, nt, tiles, pre, [](int) { return false; }, wave, wm, wn, lane);
  }

  // skip(t) (wave-uniform) lets a wave leave out the products of tile t when they are known to
  // be zero for its fragments; copies and barriers still run for the whole block.
  template <class Tiles, class Pre, class Skip>
  __device__ __forceinline__ void run(u32x4* lds, int nt, Tiles&& tiles, Pre&& pre, Skip&& skip,
                                      int wave, int wm, int wn, int lane) {
    pipeline(lds, nt, tiles,
             [&](int t, const u32x4* stage) {
               pre(t);
               if (!skip(t)) compute(stage, wm, wn, lane);
             },
             wave, lane);
  }

  // The copy pipeline alone: body(t, stage) consumes K-tile t from its LDS stage (e.g. into the
  // accumulators of another TileGemm of the same shape). Returns with every copy complete and
  // every wave past a final barrier, so LDS may be reused.
  template <class Tiles, class Body>
  __device__ __forceinline__ static void pipeline(u32x4* lds, int nt, Tiles&& tiles, Body&& body,
                                                  int wave, int lane) {
    if (nt <= 0) return;
    if constexpr (NS == 2 && SB) {
      issue_tile(lds, tiles, 0, wave, lane);
      for (int t = 0; t < nt; ++t) {
        wait_vm<0>();     // this wave's copies of tile t are done (nothing else is in flight)
        __syncthreads();  // tile t is in LDS for every wave; every wave is done with tile t-1
        if (t + 1 < nt) issue_tile(lds, tiles, t + 1, wave, lane);
        body(t, lds + (t % NS) * kStage);
      }
      __syncthreads();
      return;
    }
    issue_tile(lds, tiles, 0, wave, lane);
    if (nt > 1) issue_tile(lds, tiles, 1, wave, lane);
    for (int t = 0; t < nt; ++t) {
      // this wave's copies of tile t are done when at most those of tile t+1 are in flight
      if (t + 1 < nt)
        wait_vm<IPW>();
      else
        wait_vm<0>();
      __syncthreads();  // tile t is in LDS for every wave
      if constexpr (NS == 3) {
        // stage (t+2)%3 held tile t-1, which every wave finished before the barrier above
        if (t + 2 < nt) issue_tile(lds, tiles, t + 2, wave, lane);
      }
      body(t, lds + (t % NS) * kStage);
      if constexpr (NS == 2) {
        __syncthreads();  // every wave is done with stage t%2
        if (t + 2 < nt) issue_tile(lds, tiles, t + 2, wave, lane);
      }
    }
    if constexpr (NS == 3) __syncthreads();
  }

  // Output staging for results whose memory layout is contiguous along the tile's rows (the
  // four consecutive rows a lane holds): conv(i, j, row, col, acc, out) returns in out the four
  // output values of the lane's part of fragment (i, j), whose first row is row and column col,
  // (already rounded to the element type T); they are written to this wave's LDS
  // region as [col][row] rows of WTM elements (16-byte chunks XOR-swizzled by col), read back
  // as 16-byte chunks and handed to emit(col, row, chunk) with row a multiple of 16/sizeof(T).
  // Consecutive lanes then cover whole rows, so global stores are full 16-byte runs. The LDS
  // tile stages must be idle (after run() returns) and each wave only touches its own region.
  template <class T, class Conv, class Emit>
  __device__ __forceinline__ void stage_rows(u32x4* lds, int wave, int wm, int wn, int lane,
                                             Conv&& conv, Emit&& emit) const {
    constexpr int kCpr = WTM * int(sizeof(T)) / 16;  // 16-byte chunks per staged row
    constexpr int kRegionBytes = WTM * WTN * int(sizeof(T));
    static_assert(kCpr >= 1 && (kCpr & (kCpr - 1)) == 0, "staged row must be 2^k chunks");
    // The 16 columns one write instruction covers start kCpr*16 bytes apart; kPer of them share a
    // 256-byte bank period, so the chunk swizzle takes col / kPer: the 16 rows' chunks then fall in
    // distinct banks.
    constexpr int kPer = kCpr >= 16 ? 1 : 16 / kCpr;
    static_assert(WM * WN * kRegionBytes <= kLds * 16, "staging regions exceed the LDS tiles");
    char* region = reinterpret_cast<char*>(lds) + wave * kRegionBytes;
    const int lr = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = i * 16 + q * 4;  // wave-local
        const int col = j * 16 + lr;
        T v[4];
        conv(i, j, wm * WTM + row, wn * WTN + col, acc[i][j], v);
        const int byte = row * int(sizeof(T));
        char* dst = region + col * (kCpr * 16) + (((byte >> 4) ^ ((col / kPer) & (kCpr - 1))) << 4) + (byte & 15);
        if constexpr (sizeof(T) == 2) {
          u32x2 w;
          w[0] = uint32_t(v[0]) | (uint32_t(v[1]) << 16);
          w[1] = uint32_t(v[2]) | (uint32_t(v[3]) << 16);
          *reinterpret_cast<u32x2*>(dst) = w;
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
#pragma unroll
    for (int k = 0; k < WTN * kCpr / 64; ++k) {
      const int idx = lane + k * 64;
      const int col = idx / kCpr, ch = idx % kCpr;
      const u32x4 chunk = *reinterpret_cast<const u32x4*>(
          region + col * (kCpr * 16) + ((ch ^ ((col / kPer) & (kCpr - 1))) << 4));
      emit(wn * WTN + col, wm * WTM + ch * (16 / int(sizeof(T))), chunk);
    }
  }

  // The same for results contiguous along the tile's columns: staged as [row][col] rows of WTN
  // elements (element-wise LDS writes), handed out as emit(row, col, chunk) with col a multiple
  // of 16/sizeof(T). With PASSES > 1 the wave's rows go through its region in that many slices
  // (for wave tiles whose staged copy would not fit the LDS tiles).
  template <class T, int PASSES = 1, class Conv, class Emit>
  __device__ __forceinline__ void stage_cols(u32x4* lds, int wave, int wm, int wn, int lane,
                                             Conv&& conv, Emit&& emit) const {
    static_assert(TM % PASSES == 0, "passes split the fragment rows evenly");
    constexpr int kTMP = TM / PASSES;  // fragment rows per pass
    constexpr int kRows = kTMP * 16;
    constexpr int kCpr = WTN * int(sizeof(T)) / 16;
    constexpr int kRegionBytes = kRows * WTN * int(sizeof(T));
    static_assert(kCpr >= 1 && (kCpr & (kCpr - 1)) == 0, "staged row must be 2^k chunks");
    static_assert(WM * WN * kRegionBytes <= kLds * 16, "staging regions exceed the LDS tiles");
    char* region = reinterpret_cast<char*>(lds) + wave * kRegionBytes;
    const int lr = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
#pragma unroll
      for (int ii = 0; ii < kTMP; ++ii)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int i = ps * kTMP + ii;
          const int row = ii * 16 + q * 4;  // pass-local
          const int col = j * 16 + lr;
          T v[4];
          conv(i, j, wm * WTM + ps * kRows + row, wn * WTN + col, acc[i][j], v);
          const int byte = col * int(sizeof(T));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int rr = row + k;
            char* dst = region + rr * (kCpr * 16) + (((byte >> 4) ^ (rr & (kCpr - 1))) << 4) + (byte & 15);
            *reinterpret_cast<T*>(dst) = v[k];
          }
        }
#pragma unroll
      for (int k = 0; k < kRows * kCpr / 64; ++k) {
        const int idx = lane + k * 64;
        const int row = idx / kCpr, ch = idx % kCpr;
        const u32x4 chunk = *reinterpret_cast<const u32x4*>(
            region + row * (kCpr * 16) + ((ch ^ (row & (kCpr - 1))) << 4));
        emit(wm * WTM + ps * kRows + row, wn * WTN + ch * (16 / int(sizeof(T))), chunk);
      }
    }
  }

  // Calls f(row, col, acc) for each 16x16 fragment: rows row..row+3 of column col (tile-local).
  template <class F>
  __device__ __forceinline__ void epilogue(int wm, int wn, int lane, F&& f) const {
    const int lr = lane & 15;
    const int q = lane >> 4;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) f(wm * WTM + i * 16 + q * 4, wn * WTN + j * 16 + lr, acc[i][j]);
  }
};

// An epilogue's elementwise operand tile in LDS: ROWS x COLS elements of a row-major tensor (row
// pitch ld; rows past nrows and columns past ncols read as zeros) copied by THREADS threads with
// 16-byte loads that cover whole rows, each row's chunks XOR-swizzled by the row so that the 16
// rows a fragment read touches fall in distinct banks. Callers synchronise before reading it back
// with lds_tile_read4f.
template <class T, int ROWS, int COLS, int THREADS>
__device__ __forceinline__ void lds_tile_load(char* dst, const T* src, int64_t ld, int nrows,
                                              int ncols) {
  constexpr int kCpr = COLS * int(sizeof(T)) / 16;  // 16-byte chunks per row
  static_assert(kCpr >= 1 && (kCpr & (kCpr - 1)) == 0, "a tile row must be 2^k chunks");
  static_assert(ROWS * kCpr % THREADS == 0, "the chunks must spread evenly over the threads");
#pragma unroll
  for (int k = 0; k < ROWS * kCpr / THREADS; ++k) {
    const int idx = int(threadIdx.x) + k * THREADS;
    const int row = idx / kCpr, ch = idx % kCpr;
    const int col = ch * (16 / int(sizeof(T)));
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nrows && col < ncols) v = *reinterpret_cast<const u32x4*>(src + int64_t(row) * ld + col);
    *reinterpret_cast<u32x4*>(dst + row * (kCpr * 16) + ((ch ^ (row & (kCpr - 1))) << 4)) = v;
  }
}

// Elements col..col+3 of row `row` of a tile stored by lds_tile_load, as floats (col % 4 == 0).
template <class T, int COLS>
__device__ __forceinline__ void lds_tile_read4f(const char* src, int row, int col, float* o) {
  constexpr int kCpr = COLS * int(sizeof(T)) / 16;
  const int byte = col * int(sizeof(T));
  load4f(reinterpret_cast<const T*>(src + row * (kCpr * 16) +
                                    (((byte >> 4) ^ (row & (kCpr - 1))) << 4) + (byte & 15)),
         o);
}

// An MN-major operand of a TileGemm: K rows [row0, row0 + k_rows) of a row-major tensor with
// row pitch ld_elems, columns [m0, m0 + m_valid) valid (a tile reads 256 bytes of each row from
// column m0; columns past m_valid and rows past k_rows read as zeros). m_valid·esz must be a
// multiple of 16 (every dimension here is a multiple of 8).
__device__ __forceinline__ Src make_src_mn(const void* base, int64_t row0, int64_t ld_elems, int esz,
                                           int k_rows, int64_t m0, int m_valid) {
  return make_src(reinterpret_cast<const char*>(base) + m0 * esz, row0, ld_elems, esz, k_rows,
                  k_rows, m_valid);
}

struct NoPre {
  __device__ __forceinline__ void operator()(int) const {}
};

// Wave w of a workgroup runs on SIMD w % 4, so with 8 waves, waves w and w + 4 share a SIMD.
// For kernels whose work per wave grows with wn (causal key ranges), pair a short range with a
// long one on every SIMD. Other shapes use the plain row-major mapping.
template <int WM, int WN>
__device__ __forceinline__ void balanced_wave(int w, int& wm, int& wn) {
  if constexpr (WM * WN == 8 && WN == 4) {
    wm = w >> 2;
    wn = w < 4 ? w : 7 - w;
  } else if constexpr (WM * WN == 8 && WN == 2) {
    wm = w >> 1;
    wn = (w & 1) ^ ((w >> 2) & 1);
  } else {
    wm = w / WN;
    wn = w % WN;
  }
}

// ------------------------------------------------------------------------------ pack
// Transposes src [R, C] into dst [C, R] (R and C multiples of 8) without LDS: each lane moves a
// V x V block (V = 16 bytes / element size: 8 x 8 bf16 or 4 x 4 fp32) with V 16-byte row loads,
// transposes it in registers and writes V 16-byte rows. The 64 lanes of a wave cover an
// 8V x 8V tile, lane (i, j) = (lane / 8, lane % 8) the block at rows 8... of (i, j): eight lanes
// with one i read 128 contiguous bytes of a source row, eight lanes with one j write 128
// contiguous bytes of a destination row. A block lies wholly inside or wholly outside the matrix.
template <class E>
struct TransposeJob {
  const typename E::T* src;  // [R, C]
  typename E::T* dst;        // [C, R]
  int R, C;
  int tiles_c;     // wave tiles along C
  int first_tile;  // index of this job's first wave tile in the launch
};
template <class E>
struct PackArgs {
  TransposeJob<E> job[4];
  int njobs;
  int ntiles;  // wave tiles over all jobs
};

// Transposes a 8x8 block of bf16 held as 8 rows of 4 packed pairs: out row k = column k of in.
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[8], u32x4 (&out)[8], BF16) {
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int m = 0; m < 4; ++m)  // (row 2m, row 2m+1) of column k: low or high halves of pair k/2
      out[k][m] = __builtin_amdgcn_perm(in[2 * m + 1][k >> 1], in[2 * m][k >> 1],
                                        (k & 1) ? 0x07060302u : 0x05040100u);
}
__device__ __forceinline__ void transpose_block(const u32x4 (&in)[4], u32x4 (&out)[4], F32) {
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int m = 0; m < 4; ++m) out[k][m] = in[m][k];
}

template <class E>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs<E> args) {
  constexpr int V = 16 / E::kSize;  // block edge
  constexpr int TE = 8 * V;         // wave tile edge
  const int tile = int(blockIdx.x) * 4 + int(threadIdx.x >> 6);
  if (tile >= args.ntiles) return;
  int jb = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < args.njobs && tile >= args.job[i].first_tile) jb = i;
  const TransposeJob<E>& J = args.job[jb];
  const int t = tile - J.first_tile;
  const int lane = threadIdx.x & 63;
  const int r = (t / J.tiles_c) * TE + (lane >> 3) * V;  // first source row of the lane's block
  const int col = (t % J.tiles_c) * TE + (lane & 7) * V;  // first source column
  if (r >= J.R || col >= J.C) return;
  u32x4 in[V], out[V];
#pragma unroll
  for (int k = 0; k < V; ++k)
    in[k] = *reinterpret_cast<const u32x4*>(J.src + int64_t(r + k) * J.C + col);
  transpose_block(in, out, E());
#pragma unroll
  for (int k = 0; k < V; ++k)
    *reinterpret_cast<u32x4*>(J.dst + int64_t(col + k) * J.R + r) = out[k];
}

// ------------------------------------------------------------------------------ proj
// X (W_v | W_z): V and the four heads. The gate U = SiLU(X W_u) is not materialised: the mix
// stage recomputes it for its own tile, next to the product it gates.
template <class E>
struct ProjArgs {
  const typename E::T* X;     // [M, d]
  const typename E::T* WvzT;  // [e+s, d]: rows of (W_v | W_z)ᵀ
  typename E::T* Vt;          // [M/c, e, c]
  typename E::T* Qq;          // [M, s]
  typename E::T* Kq;          // [M, s]
  typename E::T* Ql;          // [M, s]
  typename E::T* Klt;         // [M/c, s, c]
  const float* gamma;         // [4, s]
  const float* beta;          // [4, s]
  int M, d, e, s, c;
  int n;             // sequence length: a token's position is its row modulo n
  int rope;          // rotate the four heads (rotary position embedding)
  double log2_base;  // log2 of the rotary base
  // Written only by the EXTRA instantiation (the backward pass recomputes the projection and
  // also needs its pre-activations):
  typename E::T* Hr;  // [M, e+s]: X W_v | X W_z before SiLU
};

template <class E, int BM, int BN, int WM, int WN, int NS, bool EXTRA = false>
__global__ __launch_bounds__(64 * WM * WN) void proj_kernel(ProjArgs<E> p) {
  using G = TileGemm<E, BM, BN, WM, WN, NS>;
  __shared__ u32x4 lds[G::kLds];
  // Columns: V (e columns), then the s head features. hcols is the row pitch of the
  // pre-activations Hr.
  const int hcols = p.e + p.s;
  const int ncols = p.e + p.s;
  const int ntn = (ncols + BN - 1) / BN;
  const int ntm = (p.M + BM - 1) / BM;
  const int lid = xcd_remap(blockIdx.x, ntm * ntn);
  int mt, nt;
  grouped_tile(lid, ntm, ntn, 8, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;

  // A tile of head features only is computed transposed (rows = features, columns = tokens):
  // each lane then holds four consecutive features of one token, so the row-major heads leave as
  // 8-byte stores and the rotary pairs sit inside the lane. The tiles are square, so swapping
  // the operands is all it takes.
  static_assert(BM == BN, "transposed head tiles need square tiles");
  const bool heads_t = n0 >= p.e;

  G g;
  g.zero();
  const Src a = make_src(p.X, m0, p.d, E::kSize, p.M - m0, BM, p.d);
  const Src b = make_src(p.WvzT, n0, p.d, E::kSize, ncols - n0, BN, p.d);
  const int nk = (p.d * E::kSize + kStageBytes - 1) / kStageBytes;
  g.run(lds, nk,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = heads_t ? b : a;
          sb = heads_t ? a : b;
          ka = kb = t * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);

  using T = typename E::T;
  const int e = p.e, s = p.s, c = p.c;
  if (heads_t) {
    g.epilogue(wm, wn, lane, [&](int r, int cl, const f32x4& v) {
      const int j = n0 - e + r;  // first of four consecutive features (s % 8 == 0)
      const int row = m0 + cl;        // token
      if (j >= s || row >= p.M) return;
      if constexpr (EXTRA) store4(p.Hr + int64_t(row) * hcols + e + j, v[0], v[1], v[2], v[3]);
      float y[4], h[4][4];  // [head][feature j + k]
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = silu(v[k]);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 4; ++k) h[q][k] = fmaf(p.gamma[q * s + j + k], y[k], p.beta[q * s + j + k]);
      if (p.rope) {
        const int pos = row % p.n;
#pragma unroll
        for (int k = 0; k < 4; k += 2) {
          float cs, sn;
          rope_angle(pos, rope_theta(j + k, s, p.log2_base), &cs, &sn);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x0 = h[q][k], x1 = h[q][k + 1];
            h[q][k] = rope_apply(x0, x1, j + k, cs, sn);
            h[q][k + 1] = rope_apply(x1, x0, j + k + 1, cs, sn);
          }
        }
      }
      const int64_t o = int64_t(row) * s + j;
      store4(p.Qq + o, h[0][0], h[0][1], h[0][2], h[0][3]);
      store4(p.Kq + o, h[1][0], h[1][1], h[1][2], h[1][3]);
      store4(p.Ql + o, h[2][0], h[2][1], h[2][2], h[2][3]);
      const int64_t bg = row / c, t = row % c;
#pragma unroll
      for (int k = 0; k < 4; ++k) p.Klt[(bg * s + j + k) * c + t] = from_f32<E>(h[3][k]);
    });
    return;
  }
  // A wave whose columns all fall in V stages its tile through LDS and writes full 16-byte runs
  // of the chunk-transposed V; other waves store element-wise.
  const int wc0 = n0 + wn * G::WTN, wc1 = wc0 + G::WTN;
  if (wc1 <= e) {
    g.template stage_rows<T>(lds, wave, wm, wn, lane,
                             [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
                               for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(silu(v[k]));
                             },
                             [&](int cl, int r, const u32x4& chunk) {
                               const int row = m0 + r, col = n0 + cl;
                               if (row >= p.M) return;
                               const int64_t bg = row / c, t = row % c;  // 8 rows, one chunk
                               store16_stream(p.Vt + (bg * e + col) * c + t, chunk);
                             });
    if constexpr (EXTRA) {
      g.template stage_cols<T>(lds, wave, wm, wn, lane,
                               [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
                                 for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
                               },
                               [&](int r, int cl, const u32x4& chunk) {
                                 const int row = m0 + r, col = n0 + cl;
                                 if (row < p.M)
                                   store16_stream(p.Hr + int64_t(row) * hcols + col, chunk);
                               });
    }
    return;
  }
  g.epilogue(wm, wn, lane, [&](int r, int cl, const f32x4& v) {
    const int row = m0 + r, gcol = n0 + cl;
    float y[4], yp[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) y[k] = silu(v[k]);
    if (p.rope) {
      // the rotary partner (feature col ^ 1, same four tokens) sits in the neighbouring lane;
      // exchanged before any lane leaves
#pragma unroll
      for (int k = 0; k < 4; ++k) yp[k] = swap_adjacent_lanes(y[k]);
    }
    if (row >= p.M || gcol >= ncols) return;
    const int64_t bg = row / c, t = row % c;  // c % 8 == 0: rows row..row+3 share a chunk
    const int col = gcol;  // V column, or e + head feature
    if constexpr (EXTRA) {
#pragma unroll
      for (int k = 0; k < 4; ++k) p.Hr[int64_t(row + k) * hcols + col] = from_f32<E>(v[k]);
    }
    if (col < e) {
      store4(p.Vt + (bg * e + col) * c + t, y[0], y[1], y[2], y[3]);
    } else {
      const int j = col - e;
      float h[4][4];  // [head][token]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float gq = p.gamma[q * s + j], bq = p.beta[q * s + j];
#pragma unroll
        for (int k = 0; k < 4; ++k) h[q][k] = fmaf(gq, y[k], bq);
      }
      if (p.rope) {
        const int jp = j ^ 1;
        const double theta = rope_theta(j, s, p.log2_base);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float cs, sn;
          rope_angle((row + k) % p.n, theta, &cs, &sn);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float partner = fmaf(p.gamma[q * s + jp], yp[k], p.beta[q * s + jp]);
            h[q][k] = rope_apply(h[q][k], partner, j, cs, sn);
          }
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t o = int64_t(row + k) * s + j;
        p.Qq[o] = from_f32<E>(h[0][k]);
        p.Kq[o] = from_f32<E>(h[1][k]);
        p.Ql[o] = from_f32<E>(h[2][k]);
      }
      store4(p.Klt + (bg * s + j) * c + t, h[3][0], h[3][1], h[3][2], h[3][3]);
    }
  });
}

// ------------------------------------------------------------------------------ scores
template <class E>
struct ScoresArgs {
  const typename E::T* Qq;  // [nbg*c, s]
  const typename E::T* Kq;  // [nbg*c, s]
  typename E::T* P;         // [nbg, c, c]
  int nbg, c, s, causal;
  float inv_c;
};

// Per chunk P = relu(Q_quad K_quadᵀ / c)², computed as Pᵀ tiles (keys x tokens) so that each
// lane holds four consecutive keys of one token and the tile leaves through LDS as 16-byte runs of
// P rows. Causal: only the tile pairs on or below the diagonal are launched (tiles entirely above
// it are never read: every wave of the mix stage skips them), and entries above the diagonal
// inside them are written as zeros.
template <class E, int BT, int WM, int WN, int NS>
__device__ __forceinline__ void scores_block(const ScoresArgs<E>& p, u32x4* lds, int bid) {
  using G = TileGemm<E, BT, BT, WM, WN, NS>;
  const int ntc = (p.c + BT - 1) / BT;
  const int per_chunk = p.causal ? ntc * (ntc + 1) / 2 : ntc * ntc;
  const int lid = xcd_remap(bid, p.nbg * per_chunk);
  const int bg = lid / per_chunk;
  const int rem = lid % per_chunk;
  int tt, kt;  // token tile, key tile
  if (p.causal) {
    // rem = tt (tt + 1) / 2 + kt with 0 <= kt <= tt
    tt = int((sqrtf(8.0f * float(rem) + 1.0f) - 1.0f) * 0.5f);
    while (tt * (tt + 1) / 2 > rem) --tt;
    while ((tt + 1) * (tt + 2) / 2 <= rem) ++tt;
    kt = rem - tt * (tt + 1) / 2;
  } else {
    tt = rem / ntc;
    kt = rem % ntc;
  }
  const int k0 = kt * BT, t0 = tt * BT;  // m: key, n: token
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;

  G g;
  g.zero();
  const int64_t base = int64_t(bg) * p.c;
  const Src a = make_src(p.Kq, base + k0, p.s, E::kSize, p.c - k0, BT, p.s);
  const Src b = make_src(p.Qq, base + t0, p.s, E::kSize, p.c - t0, BT, p.s);
  const int nk = (p.s * E::kSize + kStageBytes - 1) / kStageBytes;
  g.run(lds, nk,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = b;
          ka = kb = t * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);
  using T = typename E::T;
  T* P = p.P + base * p.c;
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int r, int cl, const f32x4& v, T* out) {
        const int key = k0 + r, tok = t0 + cl;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x = fmaxf(v[k] * p.inv_c, 0.0f);
          out[k] = from_f32<E>((p.causal && key + k > tok) ? 0.0f : x * x);
        }
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int key = k0 + r, tok = t0 + cl;
        if (key < p.c && tok < p.c) store16_stream(P + int64_t(tok) * p.c + key, chunk);
      });
}

// ------------------------------------------------------------------------------ states
// The n/c chunks of a sequence are split into ng groups of gs consecutive chunks; one workgroup
// owns (sequence, chunk group, state-row tile, value-column tile) and runs its accumulator over
// the group's chunks in order, so the accumulator is the exclusive prefix inside the group when
// each chunk starts. The group total goes to the carry buffer; the carry stage adds the totals of
// earlier groups.
template <class E>
struct StatesArgs {
  const typename E::T* Klt;  // [B*G, s, c]
  const typename E::T* Vt;   // [B*G, e, c]
  typename E::T* St;         // causal [B*G, e, s], non-causal [B, e, s]
  typename E::T* Carry;      // [B, ng, e, s]
  int B, G, s, e, c, causal;
  int ng, gs;
  float inv_n;
  // rev = 1 walks the chunks of each sequence last to first: the exclusive prefix becomes the sum
  // over the LATER chunks (the backward pass's state gradients); chunk g is stored at G-1-g.
  int rev;
};

// L = kLayoutMN reads K_lin and V token-major ([tokens, s] and [tokens, e] behind the Klt and Vt
// pointers) instead of chunk-transposed.
template <class E, int BM, int BN, int WM, int WN, int NS, int L = kLayoutK>
__device__ __forceinline__ void states_block(const StatesArgs<E>& p, u32x4* lds, int bid) {
  using G = TileGemm<E, BM, BN, WM, WN, NS, false, 1, L, L>;
  const int nts = (p.s + BM - 1) / BM;
  const int nte = (p.e + BN - 1) / BN;
  const int lid = xcd_remap(bid, p.B * p.ng * nts * nte);
  // neighbouring workgroups share a chunk group, hence its K_lin and V rows
  const int nt = lid % nte;
  int rest = lid / nte;
  const int mt = rest % nts;
  rest /= nts;
  const int grp = rest % p.ng;
  const int b = rest / p.ng;
  const int m0 = mt * BM, n0 = nt * BN;  // m: state row (s), n: value column (e)
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;

  const int nk = (p.c * E::kSize + kStageBytes - 1) / kStageBytes;
  const int g0 = grp * p.gs;
  const int nchunks = min(p.G, g0 + p.gs) - g0;
  // Causal: the sequence's last chunk in walking order feeds no state (its summary would only be
  // added after the last prefix is taken), so the last group leaves its K_lin and V unread.
  const bool last_causal = p.causal && grp == p.ng - 1;
  const int nsum = last_causal ? nchunks - 1 : nchunks;
  const int64_t chunk0 = int64_t(b) * p.G + g0;
  // storage index of the sequence's chunk chunk0 + k (k counted in walking order)
  auto phys = [&](int64_t k) -> int64_t {
    return p.rev ? int64_t(b) * p.G + (p.G - 1 - (g0 + k)) : chunk0 + k;
  };

  auto write_state = [&](G& gg, typename E::T* dst) __attribute__((always_inline)) {
    gg.epilogue(wm, wn, lane, [&](int r, int cl, const f32x4& v) {
      const int i = m0 + r, j = n0 + cl;
      if (i >= p.s || j >= p.e) return;
      store4(dst + int64_t(j) * p.s + i, v[0] * p.inv_n, v[1] * p.inv_n, v[2] * p.inv_n,
             v[3] * p.inv_n);
    });
  };
  const int64_t es = int64_t(p.e) * p.s;
  const bool write_local = p.causal && (p.gs > 1 || p.ng == 1);

  G g;
  g.zero();
  if (nsum == 0 && !(last_causal && write_local)) return;
  g.run(lds, nsum * nk,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          const int64_t chunk = phys(t / nk);
          if constexpr (L == kLayoutK) {
            sa = make_src(p.Klt, chunk * p.s + m0, p.c, E::kSize, p.s - m0, BM, p.c);
            sb = make_src(p.Vt, chunk * p.e + n0, p.c, E::kSize, p.e - n0, BN, p.c);
            ka = kb = (t % nk) * kStageBytes;
          } else {
            sa = make_src_mn(p.Klt, chunk * p.c, p.s, E::kSize, p.c, m0, p.s - m0);
            sb = make_src_mn(p.Vt, chunk * p.c, p.e, E::kSize, p.c, n0, p.e - n0);
            ka = kb = (t % nk) * G::KS;
          }
        },
        [&](int t) {
          // exclusive prefix inside the group: chunk g reads the group's chunks before it. With
          // one chunk per group that prefix is zero; the carry stage then writes every state
          // (unless there is only one group, i.e. one chunk).
          if (write_local && t % nk == 0) write_state(g, p.St + phys(t / nk) * es);
        },
        wave, wm, wn, lane);
  if (last_causal) {
    // the prefix of the group's last chunk (inside the group) is the accumulator now; the last
    // group's total is never read
    if (write_local) write_state(g, p.St + phys(nchunks - 1) * es);
    return;
  }
  // The final tile leaves through LDS (the stages are idle now) as 16-byte runs along s.
  auto write_final = [&](typename E::T* dst) {
    using T = typename E::T;
    g.template stage_rows<T>(
        lds, wave, wm, wn, lane,
        [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
          for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k] * p.inv_n);
        },
        [&](int cl, int r, const u32x4& chunk) {
          const int i = m0 + r, j = n0 + cl;
          if (i < p.s && j < p.e) *reinterpret_cast<u32x4*>(dst + int64_t(j) * p.s + i) = chunk;
        });
  };
  if (!p.causal && p.ng == 1)
    write_final(p.St + int64_t(b) * es);
  else
    write_final(p.Carry + (int64_t(b) * p.ng + grp) * es);
}

// ------------------------------------------------------------------------------ scores + states
// The per-chunk scores and the chunk summaries read only the projection's outputs, so one launch
// runs both: workgroups [0, n_scores) compute score tiles, the rest summary tiles. The memory-bound
// summaries overlap the scores instead of waiting for their last wave. n_scores is a multiple of
// the XCD count, so both ranges keep their XCD-aware tile order (extra score workgroups return).
template <class E, class S>
__global__ __launch_bounds__(64 * S::kScoresWM * S::kScoresWN) void scores_states_kernel(
    ScoresArgs<E> sp, int n_scores, int scores_blocks, StatesArgs<E> tp, int states_on) {
  static_assert(S::kScoresWM * S::kScoresWN == S::kStatesWM * S::kStatesWN,
                "both roles run with the same workgroup size");
  using GS = TileGemm<E, S::kScoresBT, S::kScoresBT, S::kScoresWM, S::kScoresWN, S::kScoresNS>;
  using GT = TileGemm<E, S::kStatesBM, S::kStatesBN, S::kStatesWM, S::kStatesWN, S::kStatesNS>;
  __shared__ u32x4 lds[GS::kLds > GT::kLds ? GS::kLds : GT::kLds];
  const int bid = blockIdx.x;
  if (bid < n_scores) {
    if (bid < scores_blocks)
      scores_block<E, S::kScoresBT, S::kScoresWM, S::kScoresWN, S::kScoresNS>(sp, lds, bid);
  } else if (states_on) {
    states_block<E, S::kStatesBM, S::kStatesBN, S::kStatesWM, S::kStatesWN, S::kStatesNS>(
        tp, lds, bid - n_scores);
  }
}

// ------------------------------------------------------------------------------ carry
template <class E>
struct CarryArgs {
  typename E::T* St;           // causal [B*G, e, s], non-causal [B, e, s]
  const typename E::T* Carry;  // [B, ng, e, s]
  int B, G, ng, gs, causal;
  int64_t es;                  // e * s, a multiple of 8
  int rev;                     // chunks walked last to first (as in StatesArgs)
};

__device__ __forceinline__ void load8(const uint16_t* p, float* o) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[2 * k] = __uint_as_float(v[k] << 16);
    o[2 * k + 1] = __uint_as_float(v[k] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* o) {
  const f32x4 a = reinterpret_cast<const f32x4*>(p)[0], b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    o[k] = a[k];
    o[4 + k] = b[k];
  }
}
__device__ __forceinline__ void store8(uint16_t* p, const float* v) {
  u32x4 w;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    w[k] = uint32_t(f32_to_bf16(v[2 * k])) | (uint32_t(f32_to_bf16(v[2 * k + 1])) << 16);
  store16_stream(p, w);
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  reinterpret_cast<f32x4*>(p)[0] = f32x4{v[0], v[1], v[2], v[3]};
  reinterpret_cast<f32x4*>(p)[1] = f32x4{v[4], v[5], v[6], v[7]};
}

// The carry walk of 8 consecutive elements (offset j inside one [e, s] state) of sequence b, over
// the chunk groups in order. Chunk and group totals are loaded kCarryBatch at a time ahead of
// their sums, so that the loads' latencies overlap; the sums keep the walking order.
constexpr int kCarryBatch = 8;

template <class E>
__device__ __forceinline__ void carry_vec(const CarryArgs<E>& p, int b, int64_t j) {
  float run[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const typename E::T* tot = p.Carry + int64_t(b) * p.ng * p.es + j;
  auto chunk_at = [&](int g) -> int64_t { return int64_t(b) * p.G + (p.rev ? p.G - 1 - g : g); };
  if (p.causal && p.gs == 1) {
    // one chunk per group: the states stage left only the chunk totals (of chunks 0..G-2); write
    // the exclusive prefix of every chunk directly
    for (int g0 = 0; g0 < p.G; g0 += kCarryBatch) {
      float v[kCarryBatch][8];
#pragma unroll
      for (int q = 0; q < kCarryBatch; ++q)
        if (g0 + q < p.G - 1) load8(tot + int64_t(g0 + q) * p.es, v[q]);
#pragma unroll
      for (int q = 0; q < kCarryBatch; ++q) {
        if (g0 + q >= p.G) break;
        store8(p.St + chunk_at(g0 + q) * p.es + j, run);
        if (g0 + q < p.G - 1) {
#pragma unroll
          for (int k = 0; k < 8; ++k) run[k] += v[q][k];
        }
      }
    }
  } else if (p.causal) {
    // the states stage left each chunk's prefix inside its group; add the earlier groups' totals
    float v[8];
    for (int k = 0; k < p.ng; ++k) {
      if (k > 0) {
        const int g1 = min(p.G, (k + 1) * p.gs);
        for (int g = k * p.gs; g < g1; ++g) {
          typename E::T* ptr = p.St + chunk_at(g) * p.es + j;
          load8(ptr, v);
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += run[q];
          store8(ptr, v);
        }
      }
      if (k < p.ng - 1) {
        load8(tot + int64_t(k) * p.es, v);
#pragma unroll
        for (int q = 0; q < 8; ++q) run[q] += v[q];
      }
    }
  } else {
    for (int k0 = 0; k0 < p.ng; k0 += kCarryBatch) {
      float v[kCarryBatch][8];
#pragma unroll
      for (int q = 0; q < kCarryBatch; ++q)
        if (k0 + q < p.ng) load8(tot + int64_t(k0 + q) * p.es, v[q]);
#pragma unroll
      for (int q = 0; q < kCarryBatch; ++q) {
        if (k0 + q >= p.ng) break;
#pragma unroll
        for (int k = 0; k < 8; ++k) run[k] += v[q][k];
      }
    }
    store8(p.St + int64_t(b) * p.es + j, run);
  }
}

// One thread per 8 consecutive state elements of one sequence.
template <class E>
__global__ __launch_bounds__(256) void carry_kernel(CarryArgs<E> p) {
  const int64_t per_seq = p.es / 8;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= p.B * per_seq) return;
  carry_vec(p, int(idx / per_seq), (idx % per_seq) * 8);
}

// ------------------------------------------------------------------------------ mix
template <class E>
struct MixArgs {
  const typename E::T* Vt;   // [B*G, e, c]
  const typename E::T* St;   // causal [B*G, e, s], non-causal [B, e, s]
  const typename E::T* P;    // [B*G, c, c]
  const typename E::T* Ql;   // [B*G*c, s]
  const typename E::T* X;    // [B*G*c, d]
  const typename E::T* WuT;  // [e, d]: rows of W_uᵀ
  typename E::T* Y;          // [B*G*c, e]
  int d;
  int nbg, G, c, e, s, causal;
  int lin;  // 0: no global term (causal with a single chunk: its prefix state is empty)
  typename E::T* Hu;  // HU instantiation (the training forward): X W_u before SiLU, [B*G*c, e],
                      // written here for the backward
};

template <class E, int BM, int BN, int WM, int WN, int NS, bool HU = false>
__global__ __launch_bounds__(64 * WM * WN) void mix_kernel(MixArgs<E> p) {
  using G = TileGemm<E, BM, BN, WM, WN, NS>;
  __shared__ u32x4 lds[G::kLds];
  const int nte = (p.e + BM - 1) / BM;
  const int ntt = (p.c + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, p.nbg * nte * ntt);
  const int bg = lid / (nte * ntt);
  const int rem = lid % (nte * ntt);
  const int nt = rem / nte, mt = rem % nte;
  const int m0 = mt * BM, n0 = nt * BN;  // m: value column (e), n: token inside the chunk
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  int wm, wn;
  balanced_wave<WM, WN>(wave, wm, wn);

  // Causal: tokens n0..n0+BN-1 attend to keys 0..n0+BN-1 of their chunk only; P is zero above
  // the diagonal, so stopping the key range there is exact. Inside the block, a wave whose
  // tokens all precede a key tile skips that tile's products.
  const int keys = p.causal ? min(p.c, n0 + BN) : p.c;
  const int nk0 = (keys * E::kSize + kStageBytes - 1) / kStageBytes;
  const int nk1 = p.lin ? (p.s * E::kSize + kStageBytes - 1) / kStageBytes : 0;
  const int64_t tok0 = int64_t(bg) * p.c;
  const int64_t slot = p.causal ? bg : bg / p.G;
  const Src a0 = make_src(p.Vt, int64_t(bg) * p.e + m0, p.c, E::kSize, p.e - m0, BM, p.c);
  const Src b0 = make_src(p.P, tok0 + n0, p.c, E::kSize, p.c - n0, BN, p.c);
  const Src a1 = make_src(p.St, slot * p.e + m0, p.s, E::kSize, p.e - m0, BM, p.s);
  const Src b1 = make_src(p.Ql, tok0 + n0, p.s, E::kSize, p.c - n0, BN, p.s);

  constexpr int kKeysPerTile = kStageBytes / E::kSize;
  const int last_token = n0 + (wn + 1) * G::WTN - 1;  // of this wave

  // The gate first: Uᵀ = W_uᵀ Xᵀ for these value columns and tokens, a GEMM over d into its own
  // accumulators (the projection stage does not write U); then the local and the global term.
  // Two pipelines one after the other keep the kernel within 128 registers, so two workgroups
  // share a CU (one pipeline over all three K-ranges needs more and halves the occupancy).
  G gu;
  gu.zero();
  {
    const Src au = make_src(p.WuT, m0, p.d, E::kSize, p.e - m0, BM, p.d);
    const Src bu = make_src(p.X, tok0 + n0, p.d, E::kSize, p.c - n0, BN, p.d);
    const int nku = (p.d * E::kSize + kStageBytes - 1) / kStageBytes;
    gu.run(lds, nku,
           [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
             sa = au;
             sb = bu;
             ka = kb = t * kStageBytes;
           },
           NoPre(), wave, wm, wn, lane);
  }

  G g;
  g.zero();
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

  // Y = SiLU(X W_u) ⊙ (P V + Q_lin S / n), formed in fp32 from both accumulators, rounded once,
  // and staged through LDS so that every token row of Y is written as full 16-byte runs. The
  // training forward (HU) first writes the gate's pre-activations H_u the same way, rounded to the
  // storage type, and forms Y from the rounded values: the backward's recompute reads that same
  // H_u, so both arrive at the same Y.
  using T = typename E::T;
  if constexpr (HU) {
    gu.template stage_rows<T>(
        lds, wave, wm, wn, lane,
        [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
          for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
        },
        [&](int cl, int r, const u32x4& chunk) {
          const int j = m0 + r, i = n0 + cl;
          if (j < p.e && i < p.c) store16_stream(p.Hu + (tok0 + i) * p.e + j, chunk);
        });
#pragma unroll
    for (int i = 0; i < G::TM; ++i)
#pragma unroll
      for (int j = 0; j < G::TN; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) gu.acc[i][j][k] = to_f32(from_f32<E>(gu.acc[i][j][k]));
  }
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int fi, int fj, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(silu(gu.acc[fi][fj][k]) * v[k]);
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int j = m0 + r, i = n0 + cl;
        if (j < p.e && i < p.c) store16_stream(p.Y + (tok0 + i) * p.e + j, chunk);
      });
}

// ------------------------------------------------------------------------------ out
template <class E>
struct OutArgs {
  const typename E::T* WoT;  // [d, e]
  const typename E::T* Y;    // [M, e]
  typename E::T* O;          // [M, d]
  int M, d, e;
};

template <class E, int BM, int BN, int WM, int WN, int NS, bool PRIO, bool SB = false>
__global__ __launch_bounds__(64 * WM * WN) void out_kernel(OutArgs<E> p) {
  using G = TileGemm<E, BM, BN, WM, WN, NS, PRIO, 1, kLayoutK, kLayoutK, SB>;
  __shared__ u32x4 lds[G::kLds];
  const int ntd = (p.d + BM - 1) / BM;
  const int ntt = (p.M + BN - 1) / BN;
  const int lid = xcd_remap(blockIdx.x, ntd * ntt);
  const int nt = lid / ntd, mt = lid % ntd;
  const int m0 = mt * BM, n0 = nt * BN;  // m: output feature (d), n: token
  const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
  const int wm = wave / WN, wn = wave % WN;

  G g;
  g.zero();
  const Src a = make_src(p.WoT, m0, p.e, E::kSize, p.d - m0, BM, p.e);
  const Src b = make_src(p.Y, n0, p.e, E::kSize, p.M - n0, BN, p.e);
  const int nk = (p.e * E::kSize + kStageBytes - 1) / kStageBytes;
  g.run(lds, nk,
        [&](int t, Src& sa, int& ka, Src& sb, int& kb) {
          sa = a;
          sb = b;
          ka = kb = t * kStageBytes;
        },
        NoPre(), wave, wm, wn, lane);
  using T = typename E::T;
  g.template stage_rows<T>(
      lds, wave, wm, wn, lane,
      [&](int, int, int, int, const f32x4& v, T* out) {
#pragma unroll
        for (int k = 0; k < 4; ++k) out[k] = from_f32<E>(v[k]);
      },
      [&](int cl, int r, const u32x4& chunk) {
        const int j = m0 + r, i = n0 + cl;  // j: first of the chunk's features, i: token
        if (j < p.d && i < p.M) store16_stream(p.O + int64_t(i) * p.d + j, chunk);
      });
}

// ------------------------------------------------------------------------------ tile shapes
// (BM, BN, waves along M, waves along N[, register prefetch depth]) per kernel and element type.
// The two large GEMMs run 8 waves per block: a single wave per SIMD cannot issue matrix
// instructions back to back, two can.
template <class E> struct Shapes;
template <> struct Shapes<BF16> {
  static constexpr int kProjBM = 128, kProjBN = 128, kProjWM = 2, kProjWN = 4, kProjNS = 2;
  static constexpr int kScoresBT = 128, kScoresWM = 2, kScoresWN = 4, kScoresNS = 2;
  // states and mix: 64 KB of LDS, so two blocks share a CU and one's epilogue overlaps the
  // other's loads
  static constexpr int kStatesBM = 128, kStatesBN = 128, kStatesWM = 2, kStatesWN = 4;
  static constexpr int kStatesNS = 2;
  static constexpr int kMixBM = 128, kMixBN = 128, kMixWM = 2, kMixWN = 4, kMixNS = 2;
  static constexpr int kOutBM = 256, kOutBN = 128, kOutWM = 4, kOutWN = 2, kOutNS = 3;
  static constexpr bool kOutPrio = true;
  // the output GEMM's large tile (256 x 256, 8 waves of 128 x 64, single-barrier two-stage ring),
  // taken when its tile count fills the CUs' rounds better (launch_out)
  static constexpr bool kOutBig = true;
};
// fp32's matrix rate is a sixteenth of bf16's, so its tiles can be small without the LDS becoming
// the limit: 32 x 32 projection and output tiles, 32 (value columns) x 64 (tokens) mix tiles and
// 64 x 64 state tiles spread a call's work over many more workgroups than 128 x 128 tiles do (the
// fp32 configuration, B = 1, n = 512, gave its output GEMM 8 workgroups with those).
template <> struct Shapes<F32> {
  static constexpr int kProjBM = 32, kProjBN = 32, kProjWM = 2, kProjWN = 2, kProjNS = 3;
  static constexpr int kScoresBT = 64, kScoresWM = 2, kScoresWN = 2, kScoresNS = 3;
  static constexpr int kStatesBM = 64, kStatesBN = 64, kStatesWM = 2, kStatesWN = 2;
  static constexpr int kStatesNS = 3;
  static constexpr int kMixBM = 32, kMixBN = 64, kMixWM = 2, kMixWN = 2, kMixNS = 3;
  static constexpr int kOutBM = 32, kOutBN = 32, kOutWM = 2, kOutWN = 2, kOutNS = 3;
  static constexpr bool kOutPrio = false;
  static constexpr bool kOutBig = false;
};

// The scores stage leaves P tiles entirely above the diagonal unwritten. The mix stage never
// multiplies them as long as each of its token tiles is one scores token tile (so a wave's tokens
// all lie in one scores tile) and its key tiles nest in the scores key tiles.
template <class E>
constexpr bool scores_cover_mix() {
  using S = Shapes<E>;
  return S::kScoresBT == S::kMixBN && S::kScoresBT % (kStageBytes / E::kSize) == 0;
}
static_assert(scores_cover_mix<BF16>() && scores_cover_mix<F32>(),
              "unwritten causal P tiles could be read by the mix stage");


// ------------------------------------------------------------------------------ host side
struct Plan {
  int64_t B, n, d, e, s, c, G, M, nbg, ncols;
  int64_t ng, gs;  // chunk groups per sequence in the states stage, chunks per group
  int64_t esz;
  size_t off[FLASHGAU_WS_COUNT];
  size_t total;
};

// largest score buffer B*n*chunk (elements) the forward materialises
constexpr int64_t kMaxScoreElems = int64_t(1) << 33;

// states tile (both element types) and the workgroup count the chunk grouping aims for
constexpr int64_t kStatesTargetBlocks = 2048;

// The states stage's tile (state rows x value columns) for an element size.
inline void states_tile(int64_t esz, int64_t* tm, int64_t* tn) {
  *tm = esz == 2 ? Shapes<BF16>::kStatesBM : Shapes<F32>::kStatesBM;
  *tn = esz == 2 ? Shapes<BF16>::kStatesBN : Shapes<F32>::kStatesBN;
}

int make_plan(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk, int causal,
              flashgau_dtype dtype, Plan* p) {
  if (dtype != FLASHGAU_F32 && dtype != FLASHGAU_BF16) return FLASHGAU_ERR_UNSUPPORTED;
  if (B < 0 || n < 0 || d < 1 || e < 1 || s < 1 || chunk < 1) return FLASHGAU_ERR_BAD_SHAPE;
  if (n % chunk != 0) return FLASHGAU_ERR_BAD_SHAPE;
  if (d % 8 || e % 8 || s % 8 || chunk % 8) return FLASHGAU_ERR_UNSUPPORTED;
  memset(p, 0, sizeof(*p));
  p->B = B; p->n = n; p->d = d; p->e = e; p->s = s; p->c = chunk;
  p->esz = dtype == FLASHGAU_BF16 ? 2 : 4;
  int64_t M;
  if (!mul_ok(B, n, &M) || M > kInt32Max) return FLASHGAU_ERR_BAD_SHAPE;
  p->M = M;
  p->G = chunk > 0 ? n / chunk : 0;
  p->nbg = B * p->G;
  p->ncols = 2 * e + s;
  if (d > kInt32Max || p->ncols > kInt32Max || chunk > kInt32Max) return FLASHGAU_ERR_BAD_SHAPE;
  // About two thousand states workgroups: enough chunk groups to fill the chip many times over.
  {
    int64_t tm, tn;
    states_tile(p->esz, &tm, &tn);
    const int64_t base = B * cdiv(s, tm) * cdiv(e, tn);
    int64_t ng = base > 0 ? cdiv(kStatesTargetBlocks, base) : 1;
    ng = std::max<int64_t>(1, std::min<int64_t>(ng, std::max<int64_t>(p->G, 1)));
    p->gs = p->G > 0 ? cdiv(p->G, ng) : 1;
    p->ng = p->G > 0 ? cdiv(p->G, p->gs) : 1;
  }
  if (M == 0) {
    p->total = 0;
    return FLASHGAU_OK;
  }
  // Element counts of each buffer; every product is checked.
  int64_t cnt[FLASHGAU_WS_COUNT];
  int64_t t0;
  if (!mul_ok(p->ncols, d, &cnt[FLASHGAU_WS_WCAT_T])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(d, e, &cnt[FLASHGAU_WS_WO_T])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(M, e, &cnt[FLASHGAU_WS_VT])) return FLASHGAU_ERR_BAD_SHAPE;
  if (!mul_ok(M, s, &cnt[FLASHGAU_WS_QQ])) return FLASHGAU_ERR_BAD_SHAPE;
  cnt[FLASHGAU_WS_KQ] = cnt[FLASHGAU_WS_QL] = cnt[FLASHGAU_WS_KLT] = cnt[FLASHGAU_WS_QQ];
  if (!mul_ok(M, chunk, &cnt[FLASHGAU_WS_P])) return FLASHGAU_ERR_BAD_SHAPE;
  // Every chunk's c x c scores are kept in HBM; past 2^33 of them (16 GiB in bf16, e.g. one
  // sequence of 131072 tokens as a single chunk) a shorter chunk is the layer to run.
  if (cnt[FLASHGAU_WS_P] > kMaxScoreElems) return FLASHGAU_ERR_UNSUPPORTED;
  if (!mul_ok(causal ? p->nbg : B, e, &t0) || !mul_ok(t0, s, &cnt[FLASHGAU_WS_ST]))
    return FLASHGAU_ERR_BAD_SHAPE;
  cnt[FLASHGAU_WS_Y] = cnt[FLASHGAU_WS_VT];
  if (!mul_ok(B * p->ng, e, &t0) || !mul_ok(t0, s, &cnt[FLASHGAU_WS_CARRY]))
    return FLASHGAU_ERR_BAD_SHAPE;
  size_t off = 0;
  for (int i = 0; i < FLASHGAU_WS_COUNT; ++i) {
    int64_t bytes;
    if (!mul_ok(cnt[i], p->esz, &bytes)) return FLASHGAU_ERR_BAD_SHAPE;
    p->off[i] = off;
    const size_t padded = (size_t(bytes) + 255) & ~size_t(255);
    if (__builtin_add_overflow(off, padded, &off)) return FLASHGAU_ERR_BAD_SHAPE;
  }
  p->total = off;
  // Grid sizes of every launch (the largest tile counts use the smallest tiles).
  // launch grids at the smallest tiles each stage takes for this dtype (bf16's smaller projection
  // and output tiles serve only problems of a few hundred tiles)
  const bool f32 = p->esz == 4;
  const int64_t pt = f32 ? Shapes<F32>::kProjBM : Shapes<BF16>::kProjBM;
  const int64_t mt = f32 ? Shapes<F32>::kMixBM : Shapes<BF16>::kMixBM;
  const int64_t mn = f32 ? Shapes<F32>::kMixBN : Shapes<BF16>::kMixBN;
  const int64_t ot = f32 ? Shapes<F32>::kOutBN : 128;
  static_assert(Shapes<F32>::kProjBM == Shapes<F32>::kProjBN && Shapes<F32>::kOutBM == Shapes<F32>::kOutBN,
                "square fp32 projection and output tiles");
  const int64_t grids[] = {
      cdiv(M, pt) * cdiv(p->ncols, pt),
      p->nbg * cdiv(chunk, 64) * cdiv(chunk, 64) + kXcds + B * p->ng * cdiv(s, 64) * cdiv(e, 64),
      cdiv(B * e * s / 8, 256),
      p->nbg * cdiv(e, mt) * cdiv(chunk, mn),
      cdiv(std::max(d, e), ot) * cdiv(M, ot),  // the output GEMM, and the backward's H_u = X W_u
  };
  for (int64_t g : grids)
    if (g > kMaxBlocks) return FLASHGAU_ERR_BAD_SHAPE;
  // the weight transposes: 64 x 64 wave tiles at bf16, 32 x 32 at fp32, four per workgroup
  const int64_t te = f32 ? 32 : 64;
  const int64_t pack_tiles = cdiv(d, te) * (2 * cdiv(e, te) + cdiv(s, te)) + cdiv(e, te) * cdiv(d, te);
  if (cdiv(pack_tiles, 4) > kMaxBlocks) return FLASHGAU_ERR_BAD_SHAPE;
  return FLASHGAU_OK;
}

// The output GEMM O = Y W_o. bf16 has two tile shapes, both one workgroup per CU: 256 (features)
// x 128 (tokens) with a three-stage ring, and 256 x 256 with a single-barrier two-stage ring,
// which does the work of two of the smaller tiles in about 1.65 times their time (measured at
// d = 768 and 1024, e = 1536 and 2048). The launch takes the shape whose tiles fill the chip's
// rounds of kCUs workgroups better: at B*n = 32768, d = 768 the small tiles make 3 full rounds
// and the large 1.5; at B*n = 16384 (d = 768) or d = 1024 the large tiles win.
constexpr int64_t kCUs = 256;  // MI355X compute units

inline bool out_big_tiles(int64_t M, int64_t d, bool big_ok) {
  if (!big_ok) return false;
  // 1.65 x the rounds of large tiles against the rounds of small tiles, in integers
  const int64_t small = cdiv(d, 256) * cdiv(M, 128), large = cdiv(d, 256) * cdiv(M, 256);
  return 100 * cdiv(large, kCUs) * 165 < 100 * 100 * cdiv(small, kCUs);
}

template <class E>
void launch_out(const OutArgs<E>& a, hipStream_t stream) {
  using S = Shapes<E>;
  if constexpr (S::kOutBig) {
    if (cdiv(a.d, 128) * cdiv(a.M, 128) < kCUs) {
      // too few even of those to give every CU one: 64 x 64 tiles of four waves (the projection's
      // small tile), four times as many workgroups again
      const int64_t nb = cdiv(a.d, 64) * cdiv(a.M, 64);
      launch_kernel((out_kernel<E, 64, 64, 2, 2, 3, false>), dim3(unsigned(nb)), dim3(256), 0,
                    stream, a);
      return;
    }
    if (cdiv(a.d, S::kOutBM) * cdiv(a.M, S::kOutBN) < kCUs) {
      // too few 256 x 128 tiles to give every CU one: 128 x 128 tiles, two per CU, twice the
      // workgroups for the same work
      const int64_t nb = cdiv(a.d, 128) * cdiv(a.M, 128);
      launch_kernel((out_kernel<E, 128, 128, 2, 4, 2, false>), dim3(unsigned(nb)), dim3(512), 0,
                         stream, a);
      return;
    }
    if (out_big_tiles(a.M, a.d, true)) {
      const int64_t nb = cdiv(a.d, 256) * cdiv(a.M, 256);
      launch_kernel((out_kernel<E, 256, 256, 2, 4, 2, false, true>), dim3(unsigned(nb)),
                         dim3(512), 0, stream, a);
      return;
    }
  }
  const int64_t nb = cdiv(a.d, S::kOutBM) * cdiv(a.M, S::kOutBN);
  launch_kernel((out_kernel<E, S::kOutBM, S::kOutBN, S::kOutWM, S::kOutWN, S::kOutNS,
                                  S::kOutPrio>),
                     dim3(unsigned(nb)), dim3(64 * S::kOutWM * S::kOutWN), 0, stream, a);
}

// The projection: bf16 on 128 x 128 tiles, two workgroups per CU, or, for a problem whose
// 128 x 128 tiles would not fill that first round of the CUs, on 64 x 64 tiles of four waves (four
// times the workgroups for the same work) with a two-stage ring (32 KB of LDS, five workgroups per
// CU, so that they all run in one round); fp32 on its own (small) tile.
template <class E, bool EXTRA = false>
void launch_proj(const ProjArgs<E>& a, hipStream_t stream) {
  using S = Shapes<E>;
  const int64_t ncols = int64_t(a.e) + a.s;
  if constexpr (S::kProjBM == 128) {
    if (cdiv(a.M, 128) * cdiv(ncols, 128) < 2 * kCUs) {
      const int64_t nb = cdiv(a.M, 64) * cdiv(ncols, 64);
      launch_kernel((proj_kernel<E, 64, 64, 2, 2, 2, EXTRA>), dim3(unsigned(nb)), dim3(256), 0,
                         stream, a);
      return;
    }
  }
  const int64_t nb = cdiv(a.M, S::kProjBM) * cdiv(ncols, S::kProjBN);
  launch_kernel(
      (proj_kernel<E, S::kProjBM, S::kProjBN, S::kProjWM, S::kProjWN, S::kProjNS, EXTRA>),
      dim3(unsigned(nb)), dim3(64 * S::kProjWM * S::kProjWN), 0, stream, a);
}

// The mix stage, one workgroup per (chunk, value-column tile, token tile). (64-column tiles of
// four waves for problems that leave CUs idle measured no faster.)
template <class E, bool HU = false>
void launch_mix(const MixArgs<E>& a, hipStream_t stream) {
  using S = Shapes<E>;
  const int64_t nb = int64_t(a.nbg) * cdiv(a.e, S::kMixBM) * cdiv(a.c, S::kMixBN);
  launch_kernel((mix_kernel<E, S::kMixBM, S::kMixBN, S::kMixWM, S::kMixWN, S::kMixNS, HU>),
                     dim3(unsigned(nb)), dim3(64 * S::kMixWM * S::kMixWN), 0, stream, a);
}

// pack: (W_u | W_v | W_z)ᵀ into WcatT [2e+s, d] and W_oᵀ into WoT [d, e], one launch.
template <class E>
void launch_pack(const void* W_u, const void* W_v, const void* W_z, const void* W_o, int d, int e,
                 int s, typename E::T* WcatT, typename E::T* WoT, hipStream_t stream) {
  using T = typename E::T;
  constexpr int TE = 8 * (16 / E::kSize);
  PackArgs<E> a;
  const int R[4] = {d, d, d, e};
  const int C[4] = {e, e, s, d};
  const T* src[4] = {reinterpret_cast<const T*>(W_u), reinterpret_cast<const T*>(W_v),
                     reinterpret_cast<const T*>(W_z), reinterpret_cast<const T*>(W_o)};
  T* dst[4] = {WcatT, WcatT + int64_t(e) * d, WcatT + int64_t(2 * e) * d, WoT};
  int tiles = 0;
  for (int i = 0; i < 4; ++i) {
    const int tr = int(cdiv(R[i], TE)), tc = int(cdiv(C[i], TE));
    a.job[i] = {src[i], dst[i], R[i], C[i], tc, tiles};
    tiles += tr * tc;
  }
  a.njobs = 4;
  a.ntiles = tiles;
  launch_kernel(pack_kernel<E>, dim3(unsigned(cdiv(tiles, 4))), dim3(256), 0, stream, a);
}

}  // namespace
