// common.h — device and host helpers shared by the library's translation units (forward,
// backward and decode): vector types, element types and conversions, SiLU, the matrix-core step, buffer
// descriptors, global-to-LDS copies, explicit memory waits, the XCD-aware tile order, and host-side
// size and pointer checks. Everything has internal linkage: each translation unit gets its own
// copy.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "flashgau.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kXcds = 8;        // MI355X: 8 accelerator complex dies, each with a private L2
constexpr int kRowChunks = 8;   // 16-byte chunks per LDS row and K-stage (128 bytes)
constexpr int kStageBytes = kRowChunks * 16;

// ------------------------------------------------------------------------------ element types
struct BF16 {
  using T = uint16_t;  // raw bf16 bits
  static constexpr int kSize = 2;
};
struct F32 {
  using T = float;
  static constexpr int kSize = 4;
};

__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }
__device__ __forceinline__ float to_f32(float v) { return v; }

// fp32 -> bf16, round to nearest even on the 16 dropped bits.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

template <class E>
__device__ __forceinline__ typename E::T from_f32(float f);
template <>
__device__ __forceinline__ uint16_t from_f32<BF16>(float f) { return f32_to_bf16(f); }
template <>
__device__ __forceinline__ float from_f32<F32>(float f) { return f; }

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

// Store four consecutive elements (8-byte aligned for bf16, 16-byte aligned for fp32).
__device__ __forceinline__ void store4(uint16_t* p, float a, float b, float c, float d) {
  u32x2 v;
  v[0] = uint32_t(f32_to_bf16(a)) | (uint32_t(f32_to_bf16(b)) << 16);
  v[1] = uint32_t(f32_to_bf16(c)) | (uint32_t(f32_to_bf16(d)) << 16);
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  f32x4 v = {a, b, c, d};
  *reinterpret_cast<f32x4*>(p) = v;
}
__device__ __forceinline__ void load4(const uint16_t* p, float* o) {
  u32x2 v = *reinterpret_cast<const u32x2*>(p);
  o[0] = __uint_as_float(v[0] << 16);
  o[1] = __uint_as_float(v[0] & 0xFFFF0000u);
  o[2] = __uint_as_float(v[1] << 16);
  o[3] = __uint_as_float(v[1] & 0xFFFF0000u);
}
__device__ __forceinline__ void load4(const float* p, float* o) {
  f32x4 v = *reinterpret_cast<const f32x4*>(p);
  o[0] = v[0];
  o[1] = v[1];
  o[2] = v[2];
  o[3] = v[3];
}

// SiLU(x) = x · sigmoid(x) ("Initial Power": Swish on U and V; read as phi_z too).
// e^{-x} is evaluated as 2^{-x·log2 e} on the hardware base-2 exponential (v_exp_f32) and the
// quotient through the hardware reciprocal (v_rcp_f32). Large negative x gives 2^{+big} = inf,
// rcp(inf) = 0 and the exact limit -0.
__device__ __forceinline__ float silu(float x) {
  const float t = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + t);
}

// d/dx [x σ(x)] = σ(x) (1 + x (1 − σ(x))); 0 and 1 in the limits (e^{-x} → inf gives σ = 0).
__device__ __forceinline__ float silu_grad(float x) {
  const float t = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  const float sg = __builtin_amdgcn_rcpf(1.0f + t);
  return sg * fmaf(x, 1.0f - sg, 1.0f);
}

// ------------------------------------------------------------------------------ matrix cores
// One 16-byte chunk per lane and operand: 8 bf16 (one 16x16x32 MFMA) or 4 fp32 (four 16x16x4
// MFMAs, component j of every lane group forming one k-slice). Lane l supplies row (l % 16) of A
// and column (l % 16) of B; lane group l / 16 selects the chunk, identically for A and B, so the
// sum over all chunks is the full contraction.
__device__ __forceinline__ void mma(f32x4& acc, const u32x4& a, const u32x4& b, BF16) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const u32x4& a, const u32x4& b, F32) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), acc, 0, 0, 0);
}

// A K-contiguous operand tile, read through a buffer resource that covers exactly its valid rows:
// the hardware range check turns every read past the last valid row into zeros, so tile loads
// need no per-lane branches. `kbytes` (a multiple of 16) is the valid length of each row; reads
// of chunks past it are sent out of range and also come back as zeros.
struct Src {
  u32x4 rsrc;   // buffer descriptor words (scalar registers)
  uint32_t ld;  // row pitch, bytes
  int kbytes;
};

// Raw buffer descriptor for gfx9-family (CDNA) parts: base address, stride 0, byte range, and
// word 3 = 32-bit data format, no swizzle.
constexpr uint32_t kBufferWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset at or past the range reads zero

// base: tensor base; row0: first row of the tile; rows: valid rows from row0 (may exceed the
// tile; only `max_rows` are ever read); k_elems: valid elements per row. Every argument is
// block-uniform; readfirstlane states that, so the descriptor lives in scalar registers.
__device__ __forceinline__ Src make_src(const void* base, int64_t row0, int64_t ld_elems, int esz,
                                        int rows, int max_rows, int k_elems) {
  Src s;
  const uint64_t addr =
      reinterpret_cast<uint64_t>(reinterpret_cast<const char*>(base) + row0 * ld_elems * esz);
  const int r = rows < 0 ? 0 : (rows > max_rows ? max_rows : rows);
  s.ld = __builtin_amdgcn_readfirstlane(uint32_t(ld_elems * esz));
  s.rsrc[0] = __builtin_amdgcn_readfirstlane(uint32_t(addr));
  s.rsrc[1] = __builtin_amdgcn_readfirstlane(uint32_t(addr >> 32) & 0xFFFFu);
  s.rsrc[2] = __builtin_amdgcn_readfirstlane(uint32_t(r) * s.ld);
  s.rsrc[3] = kBufferWord3;
  s.kbytes = __builtin_amdgcn_readfirstlane(k_elems * esz);
  return s;
}

// One wave copies 64 x 16 bytes from global memory straight into LDS (buffer_load_dwordx4 with
// the LDS destination): lane l's 16 bytes land at byte lds_addr + 16 l, out-of-range lanes write
// zeros. The load is counted in vmcnt; the caller waits for it explicitly (wait_vm) before a
// barrier makes the data visible to the other waves. M0 carries the wave-uniform LDS address.
__device__ __forceinline__ void lds_dma16(const u32x4& rsrc, uint32_t voffset, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(rsrc), "s"(lds_addr)
               : "memory");
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt left open).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (((N >> 4) & 3) << 14) | (0x7 << 4) | (0xF << 8));
}

// Rotary position embedding (the standard rotary form: the pair (x_{2k}, x_{2k+1}) of a head
// vector at position m turns by the angle m·θ_k, θ_k = base^{-2k/s}). Positions reach 2^31,
// where a float angle has lost its phase, so θ_k, m·θ_k and its reduction to [0, 2π) are
// evaluated in double precision; cos and sin of the reduced angle are taken in float.
// rope_apply rotates one pair member: x is feature j of the head, xp its partner j ^ 1.
__device__ __forceinline__ double rope_theta(int j, int s, double log2_base) {
  return exp2(-double(2 * (j >> 1)) / double(s) * log2_base);
}
__device__ __forceinline__ void rope_angle(int64_t m, double theta, float* cs, float* sn) {
  constexpr double kTwoPi = 6.283185307179586476925;
  constexpr double kInvTwoPi = 0.159154943091895335769;
  const double a = double(m) * theta;
  const double r = fma(-kTwoPi, floor(a * kInvTwoPi), a);
  sincosf(float(r), sn, cs);
}
__device__ __forceinline__ float rope_apply(float x, float xp, int j, float cs, float sn) {
  return (j & 1) ? fmaf(xp, sn, x * cs) : fmaf(x, cs, -xp * sn);
}

// Value of the neighbouring lane l ^ 1 (DPP quad permutation [1, 0, 3, 2]); every lane of the
// wave must execute it.
__device__ __forceinline__ float swap_adjacent_lanes(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// A block of consecutive rows of a row-major tensor behind a buffer descriptor that covers
// exactly its valid rows: reads past them (or at offset kOutOfRange) return zeros.
struct Rows {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t ld;  // row pitch, bytes
};
__device__ __forceinline__ Rows make_rows(const void* base, int64_t row0, int64_t ld_bytes,
                                          int valid_rows) {
  Rows r;
  const char* p = reinterpret_cast<const char*>(base) + row0 * ld_bytes;
  const int n = valid_rows < 0 ? 0 : valid_rows;
  r.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, int(n * ld_bytes), int(kBufferWord3));
  r.ld = uint32_t(ld_bytes);
  return r;
}
__device__ __forceinline__ u32x4 load16(const Rows& r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r.rsrc, off, 0, 0);
}

// A 16-byte store that streams past the caches (non-temporal). The large outputs of the GEMM
// stages are written once and read by a later launch; keeping them out of L2 leaves it to the
// operand tiles that the running kernel re-reads (measured: the projection's V part 108 -> 96
// us, the output GEMM 96 -> 88 us).
__device__ __forceinline__ void store16_stream(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Index of this wave inside its workgroup, as a scalar (every lane of a wave holds the same).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6); }

// Hardware places consecutive workgroup ids on consecutive XCDs (round robin). Give each XCD a
// contiguous range of logical tiles, so tiles that share operand rows also share an L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int xcd = bid % kXcds;
  const int local = bid / kXcds;
  const int per = nblocks / kXcds;
  const int rem = nblocks % kXcds;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

// Logical tile id -> (row tile, column tile): groups of `gm` row tiles are walked column by
// column, so the tiles in flight on one XCD share a few row blocks and a few column blocks.
__device__ __forceinline__ void grouped_tile(int lid, int ntm, int ntn, int gm, int& mt, int& nt) {
  const int per_group = gm * ntn;
  const int grp = lid / per_group;
  const int first = grp * gm;
  const int rows = min(gm, ntm - first);
  const int local = lid - grp * per_group;
  nt = local / rows;
  mt = first + local % rows;
}

// ------------------------------------------------------------------------------ host helpers
bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

constexpr int64_t kInt32Max = 2147483647;
// Launch limit: with at most 512 threads per workgroup, a grid of at most 2^22 workgroups keeps
// its work-item count within 32 bits.
constexpr int64_t kMaxBlocks = int64_t(1) << 22;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-kernel timing (the timed forward): while `g_kernel_timing` holds two events, the next launch
// made through launch_kernel records them when its kernel starts and when it ends
// (hipExtLaunchKernel) and clears them; otherwise launch_kernel is a plain launch.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local KernelTiming g_kernel_timing;

template <class... KArgs, class... Args>
void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                   hipStream_t stream, Args... args) {
  if (g_kernel_timing.start) {
    const KernelTiming t = g_kernel_timing;
    g_kernel_timing = KernelTiming{};
    hipExtLaunchKernelGGL(kernel, grid, block, uint32_t(lds_bytes), stream, t.start, t.stop, 0u,
                          args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, args...);
  }
}

// Layout of the packed weights: (W_u | W_v | W_z)ᵀ [2e+s, d], then W_oᵀ [d, e] at the next
// 256-byte boundary (the same two buffers open the forward's workspace).
int packed_plan(int64_t d, int64_t e, int64_t s, flashgau_dtype dtype, size_t* wo_off,
                size_t* total) {
  if (dtype != FLASHGAU_F32 && dtype != FLASHGAU_BF16) return FLASHGAU_ERR_UNSUPPORTED;
  if (d < 1 || e < 1 || s < 1) return FLASHGAU_ERR_BAD_SHAPE;
  if (d % 8 || e % 8 || s % 8) return FLASHGAU_ERR_UNSUPPORTED;
  const int64_t esz = dtype == FLASHGAU_BF16 ? 2 : 4;
  int64_t a, b;
  if (2 * e + s > kInt32Max || d > kInt32Max || !mul_ok(2 * e + s, d, &a) || !mul_ok(a, esz, &a) ||
      !mul_ok(d, e, &b) || !mul_ok(b, esz, &b))
    return FLASHGAU_ERR_BAD_SHAPE;
  const int64_t tiles = cdiv(d, 64) * (2 * cdiv(e, 64) + cdiv(s, 64)) + cdiv(e, 64) * cdiv(d, 64);
  if (tiles > kMaxBlocks) return FLASHGAU_ERR_BAD_SHAPE;
  const size_t pa = (size_t(a) + 255) & ~size_t(255), pb = (size_t(b) + 255) & ~size_t(255);
  *wo_off = pa;
  *total = pa + pb;
  return FLASHGAU_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

}  // namespace
