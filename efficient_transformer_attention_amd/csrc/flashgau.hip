// flashgau.hip — FLASH layer forward for AMD Instinct MI355X (gfx950, CDNA4).
//
// The layer (page "FLASH: Possibly the Most Interesting Efficient Transformer Design Recently",
// kexue.fm/archives/8934, sections "Initial Power", "Weak Attention" and "Mixed Chunk"):
//   U = SiLU(X W_u), V = SiLU(X W_v), Z = SiLU(X W_z); four scale/offset heads of Z;
//   local relu²(Q_quad K_quadᵀ / c) V inside each chunk (causal: lower triangle);
//   global Q_lin S_g / n with S_g = Σ K_lin_hᵀ V_h over all chunks (non-causal) or h < g (causal);
//   O = [U ⊙ (V̂_quad + V̂_lin)] W_o.
//
// Every contraction runs as one tiled matrix-core GEMM with its own operand sources and epilogue;
// pack and carry only move memory:
//   pack    W_u|W_v|W_z and W_o transposed so that every GEMM reads K-contiguous rows
//   proj    X [W_v|W_z]; epilogue SiLU, the four heads, V and K_lin written chunk-transposed
//   scores_states  one launch of two roles: per chunk P = relu(Q_quad K_quadᵀ / c)² (zero above
//           the diagonal when causal), and per (sequence, chunk group, tile) the chunk summaries
//           K_lin_hᵀ V_h, accumulated over the group's chunks in order so that the accumulator IS
//           the exclusive prefix inside the group (written, scaled by 1/n, before a chunk is added)
//   carry   adds the totals of earlier chunk groups to every chunk's state
//   mix     per chunk, (V̂_quad + V̂_lin)ᵀ = [V_gᵀ | S_gᵀ] [P_g | Q_lin_g]ᵀ, one GEMM with the local
//           and the global term concatenated along K, after the gate's own GEMM Uᵀ = SiLU(W_uᵀ Xᵀ)
//           for the same tile; epilogue Y = U ⊙ (·) (U never goes to memory)
//   out     O = Y W_o (computed as Oᵀ tiles so each lane stores contiguous outputs)
//
// Matrix-core mapping (CDNA4): bf16 uses v_mfma_f32_16x16x32_bf16, fp32 uses four
// v_mfma_f32_16x16x4_f32. Operand tiles are staged in LDS as rows of 128 bytes (8 chunks of 16 B);
// the 16-byte chunk index is XOR-swizzled with the row index so that both the row-wise fills and
// the fragment reads of 16 consecutive rows spread over the LDS banks. Tiles travel from global
// memory straight into a ring of two or three LDS stages (buffer loads with an LDS destination),
// so the copies of later K-tiles are in flight while one is multiplied.

#include <mutex>

#include "kernels.h"

namespace {

// ------------------------------------------------------------------ allocation-free forward
// flash_gau_forward_noalloc's workspace: a file-scope device array, one copy per GPU the library
// is loaded on, held until the process ends. In host code `scratch` names a host-side stand-in,
// never the device memory: the device address of each GPU's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The device address of the scratch copy on the device that `stream` belongs to (the null stream:
// the current device), looked up on the first call per device with that device made current for
// the lookup and the previous current device restored after it.
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess || cur < 0) return FLASHGAU_ERR_HIP;
  int dev = cur;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess || sd < 0) return FLASHGAU_ERR_HIP;
    dev = sd;
  }
  if (dev >= kMaxScratchDevices) return FLASHGAU_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return FLASHGAU_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t rc = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return FLASHGAU_ERR_HIP;
    if (rc != hipSuccess || !ptr) return FLASHGAU_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FLASHGAU_OK;
}

// packed (optional): weights already transposed by flashgau_pack_weights; the pack stage then
// launches nothing and the GEMMs read them there (wo_off: byte offset of W_oᵀ inside packed).
template <class E>
int launch_all(const Plan& pl, const void* X, const void* W_u, const void* W_v, const void* W_z,
               const float* gamma, const float* beta, const void* W_o, int causal, float rope_base,
               void* O, char* ws, hipStream_t stream, hipEvent_t const* events,
               const void* packed = nullptr, size_t wo_off = 0, bool per_kernel = false) {
  using T = typename E::T;
  using S = Shapes<E>;
  // events (optional). Boundaries (per_kernel false): events[i] is recorded right before stage i
  // is launched, and events[FLASHGAU_NUM_STAGES] after the last one. Per kernel: events[2i] and
  // events[2i + 1] record when stage i's kernel starts and ends; a stage that launches nothing
  // records both at once.
  int stage = 0;
  struct ClearTiming {  // no timing request outlives this call, whichever way it returns
    ~ClearTiming() { g_kernel_timing = KernelTiming{}; }
  } clear_timing;
  auto mark = [&]() -> bool {
    if (!events) return true;
    if (!per_kernel) return hipEventRecord(events[stage++], stream) == hipSuccess;
    if (stage > 0 && g_kernel_timing.start) {  // the stage before launched nothing
      const KernelTiming t = g_kernel_timing;
      g_kernel_timing = KernelTiming{};
      if (hipEventRecord(t.start, stream) != hipSuccess || hipEventRecord(t.stop, stream) != hipSuccess)
        return false;
    }
    if (stage < FLASHGAU_NUM_STAGES) g_kernel_timing = {events[2 * stage], events[2 * stage + 1]};
    ++stage;
    return true;
  };
  T* WcatT = packed ? reinterpret_cast<T*>(const_cast<void*>(packed))
                    : reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_WCAT_T]);
  T* WoT = packed ? reinterpret_cast<T*>(reinterpret_cast<char*>(const_cast<void*>(packed)) + wo_off)
                  : reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_WO_T]);
  T* Vt = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_VT]);
  T* Qq = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_QQ]);
  T* Kq = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_KQ]);
  T* Ql = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_QL]);
  T* Klt = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_KLT]);
  T* P = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_P]);
  T* St = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_ST]);
  T* Y = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_Y]);
  T* Carry = reinterpret_cast<T*>(ws + pl.off[FLASHGAU_WS_CARRY]);
  const int M = int(pl.M), d = int(pl.d), e = int(pl.e), s = int(pl.s), c = int(pl.c);

  if (!mark()) return FLASHGAU_ERR_HIP;
  if (!packed) launch_pack<E>(W_u, W_v, W_z, W_o, d, e, s, WcatT, WoT, stream);
  if (!mark()) return FLASHGAU_ERR_HIP;
  {
    ProjArgs<E> a{reinterpret_cast<const T*>(X), WcatT + int64_t(e) * d, Vt, Qq, Kq, Ql, Klt,
                  gamma, beta, M, d, e, s, c, int(pl.n), rope_base > 0.0f ? 1 : 0,
                  rope_base > 0.0f ? log2(double(rope_base)) : 0.0};
    launch_proj<E>(a, stream);
  }
  if (!mark()) return FLASHGAU_ERR_HIP;
  // Causal with a single chunk: the only chunk reads an empty prefix, so there is no global
  // term at all; the summary tiles and the carry stage launch nothing and ST is left unwritten.
  const bool lin = !(causal && pl.G == 1);
  {
    ScoresArgs<E> sa{Qq, Kq, P, int(pl.nbg), c, s, causal, 1.0f / float(c)};
    const int64_t ntc = cdiv(c, S::kScoresBT);
    const int64_t nsb = pl.nbg * (causal ? ntc * (ntc + 1) / 2 : ntc * ntc);
    const int64_t nsb8 = cdiv(nsb, kXcds) * kXcds;
    StatesArgs<E> ta{Klt, Vt, St, Carry, int(pl.B), int(pl.G), s, e, c, causal,
                     int(pl.ng), int(pl.gs), float(1.0 / double(pl.n)), 0};
    const int64_t ntb = lin ? pl.B * pl.ng * cdiv(s, S::kStatesBM) * cdiv(e, S::kStatesBN) : 0;
    launch_kernel((scores_states_kernel<E, S>), dim3(unsigned(nsb8 + ntb)),
                       dim3(64 * S::kScoresWM * S::kScoresWN), 0, stream, sa, int(nsb8), int(nsb), ta,
                       int(lin));
  }
  if (!mark()) return FLASHGAU_ERR_HIP;
  if (lin && pl.ng > 1) {
    CarryArgs<E> a{St, Carry, int(pl.B), int(pl.G), int(pl.ng), int(pl.gs), causal,
                   int64_t(e) * s, 0};
    const int64_t nb = cdiv(pl.B * e * s / 8, 256);
    launch_kernel(carry_kernel<E>, dim3(unsigned(nb)), dim3(256), 0, stream, a);
  }
  if (!mark()) return FLASHGAU_ERR_HIP;
  {
    MixArgs<E> a{Vt, St, P, Ql, reinterpret_cast<const T*>(X), WcatT, Y, d, int(pl.nbg),
                 int(pl.G), c, e, s, causal, int(lin)};
    launch_mix<E>(a, stream);
  }
  if (!mark()) return FLASHGAU_ERR_HIP;
  {
    OutArgs<E> a{WoT, Y, reinterpret_cast<T*>(O), M, d, e};
    launch_out<E>(a, stream);
  }
  if (!mark()) return FLASHGAU_ERR_HIP;
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

}  // namespace

extern "C" {

int flashgau_workspace_size(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk,
                            int causal, flashgau_dtype dtype, size_t* out_bytes) {
  if (!out_bytes) return FLASHGAU_ERR_NULL_PTR;
  Plan p;
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &p);
  if (rc != FLASHGAU_OK) return rc;
  *out_bytes = p.total;
  return FLASHGAU_OK;
}

size_t flashgau_workspace_bytes(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                                int64_t chunk, int causal, flashgau_dtype dtype) {
  Plan p;
  if (make_plan(B, n, d, e, s, chunk, causal, dtype, &p) != FLASHGAU_OK) return 0;
  return p.total;
}

int flashgau_workspace_offsets(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                               int64_t chunk, int causal, flashgau_dtype dtype,
                               size_t* out_offsets) {
  if (!out_offsets) return FLASHGAU_ERR_NULL_PTR;
  Plan p;
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &p);
  if (rc != FLASHGAU_OK) return rc;
  for (int i = 0; i < FLASHGAU_WS_COUNT; ++i) out_offsets[i] = p.off[i];
  return FLASHGAU_OK;
}

// The weights come either as the four matrices (W_u .. W_o) or as one packed buffer (packed,
// packed_bytes; the matrices are then ignored).
static int forward_impl(const void* X, const void* W_u, const void* W_v, const void* W_z,
                        const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                        int causal, int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                        flashgau_dtype dtype, void* O, void* workspace, size_t workspace_bytes,
                        void* hip_stream, hipEvent_t const* events, float rope_base,
                        const void* packed = nullptr, size_t packed_bytes = 0,
                        bool per_kernel = false) {
  Plan pl;
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &pl);
  if (rc != FLASHGAU_OK) return rc;
  if (!(rope_base >= 0.0f) || !std::isfinite(rope_base)) return FLASHGAU_ERR_BAD_SHAPE;
  size_t wo_off = 0, packed_total = 0;
  if (packed) {
    const int rp = packed_plan(d, e, s, dtype, &wo_off, &packed_total);
    if (rp != FLASHGAU_OK) return rp;
  }
  if (pl.M == 0) return FLASHGAU_OK;
  if (!X || !gamma || !beta || !O || !workspace) return FLASHGAU_ERR_NULL_PTR;
  if (!packed && (!W_u || !W_v || !W_z || !W_o)) return FLASHGAU_ERR_NULL_PTR;
  if (misaligned(X) || misaligned(O) || misaligned(workspace) ||
      (reinterpret_cast<uintptr_t>(gamma) & 3u) || (reinterpret_cast<uintptr_t>(beta) & 3u))
    return FLASHGAU_ERR_MISALIGNED;
  if (packed ? misaligned(packed)
             : (misaligned(W_u) || misaligned(W_v) || misaligned(W_z) || misaligned(W_o)))
    return FLASHGAU_ERR_MISALIGNED;
  if (workspace_bytes < pl.total) return FLASHGAU_ERR_WORKSPACE;
  if (packed && packed_bytes < packed_total) return FLASHGAU_ERR_WORKSPACE;
  const size_t es = size_t(pl.esz);
  const size_t nX = size_t(pl.M) * pl.d * es, nO = nX;
  const size_t nWu = size_t(pl.d) * pl.e * es, nWz = size_t(pl.d) * pl.s * es;
  const size_t nWo = size_t(pl.e) * pl.d * es, nGB = size_t(4) * pl.s * sizeof(float);
  const void* ins[] = {X, gamma, beta, packed ? packed : W_u, packed ? nullptr : W_v,
                       packed ? nullptr : W_z, packed ? nullptr : W_o};
  const size_t nin[] = {nX, nGB, nGB, packed ? packed_total : nWu, nWu, nWz, nWo};
  for (int i = 0; i < 7; ++i)
    if (overlaps(O, nO, ins[i], nin[i]) || overlaps(workspace, pl.total, ins[i], nin[i]))
      return FLASHGAU_ERR_ALIASING;
  if (overlaps(O, nO, workspace, pl.total)) return FLASHGAU_ERR_ALIASING;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  char* ws = reinterpret_cast<char*>(workspace);
  if (dtype == FLASHGAU_BF16)
    return launch_all<BF16>(pl, X, W_u, W_v, W_z, gamma, beta, W_o, causal ? 1 : 0, rope_base, O,
                            ws, stream, events, packed, wo_off, per_kernel);
  return launch_all<F32>(pl, X, W_u, W_v, W_z, gamma, beta, W_o, causal ? 1 : 0, rope_base, O,
                         ws, stream, events, packed, wo_off, per_kernel);
}

int flashgau_state_groups(int64_t B, int64_t n, int64_t d, int64_t e, int64_t s, int64_t chunk,
                          int causal, flashgau_dtype dtype, int64_t* out_groups) {
  if (!out_groups) return FLASHGAU_ERR_NULL_PTR;
  Plan p;
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &p);
  if (rc != FLASHGAU_OK) return rc;
  *out_groups = p.ng;
  return FLASHGAU_OK;
}

int flash_gau_forward(const void* X, const void* W_u, const void* W_v, const void* W_z,
                      const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                      int causal, int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                      flashgau_dtype dtype, void* O, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  return forward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                      workspace, workspace_bytes, hip_stream, nullptr, 0.0f);
}

int flash_gau_forward_packed(const void* X, const void* packed, size_t packed_bytes,
                             const float* gamma, const float* beta, int64_t chunk, int causal,
                             int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                             flashgau_dtype dtype, void* O, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  if (!packed) return FLASHGAU_ERR_NULL_PTR;
  return forward_impl(X, nullptr, nullptr, nullptr, gamma, beta, nullptr, chunk, causal, B, n, d, e,
                      s, dtype, O, workspace, workspace_bytes, hip_stream, nullptr, 0.0f, packed,
                      packed_bytes);
}

int flash_gau_forward_noalloc(const void* X, const void* W_u, const void* W_v, const void* W_z,
                              const float* gamma, const float* beta, const void* W_o,
                              int64_t chunk, int causal, int64_t B, int64_t n, int64_t d, int64_t e,
                              int64_t s, flashgau_dtype dtype, void* O, void* hip_stream) {
  Plan pl;
  const int rc = make_plan(B, n, d, e, s, chunk, causal, dtype, &pl);
  if (rc != FLASHGAU_OK) return rc;
  if (pl.M == 0) return FLASHGAU_OK;
  if (pl.total > kScratchBytes) return FLASHGAU_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int rs = scratch_for_stream(static_cast<hipStream_t>(hip_stream), &ws);
  if (rs != FLASHGAU_OK) return rs;
  return forward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                      ws, kScratchBytes, hip_stream, nullptr, 0.0f);
}

size_t flashgau_noalloc_scratch_bytes(void) { return kScratchBytes; }

int flash_gau_forward_rope(const void* X, const void* W_u, const void* W_v, const void* W_z,
                           const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                           int causal, float rope_base, int64_t B, int64_t n, int64_t d, int64_t e,
                           int64_t s, flashgau_dtype dtype, void* O, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  if (!(rope_base > 0.0f)) return FLASHGAU_ERR_BAD_SHAPE;
  return forward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                      workspace, workspace_bytes, hip_stream, nullptr, rope_base);
}

int flash_gau_forward_timed(const void* X, const void* W_u, const void* W_v, const void* W_z,
                            const float* gamma, const float* beta, const void* W_o, int64_t chunk,
                            int causal, int64_t B, int64_t n, int64_t d, int64_t e, int64_t s,
                            flashgau_dtype dtype, void* O, void* workspace,
                            size_t workspace_bytes, void* hip_stream, void* const* stage_events,
                            int num_events) {
  if (!stage_events) return FLASHGAU_ERR_NULL_PTR;
  const bool per_kernel = num_events == 2 * FLASHGAU_NUM_STAGES;
  if (num_events != FLASHGAU_NUM_STAGES + 1 && !per_kernel) return FLASHGAU_ERR_BAD_SHAPE;
  for (int i = 0; i < num_events; ++i)
    if (!stage_events[i]) return FLASHGAU_ERR_NULL_PTR;
  return forward_impl(X, W_u, W_v, W_z, gamma, beta, W_o, chunk, causal, B, n, d, e, s, dtype, O,
                      workspace, workspace_bytes, hip_stream,
                      reinterpret_cast<hipEvent_t const*>(stage_events), 0.0f, nullptr, 0,
                      per_kernel);
}

int flashgau_packed_weights_size(int64_t d, int64_t e, int64_t s, flashgau_dtype dtype,
                                 size_t* out_bytes) {
  if (!out_bytes) return FLASHGAU_ERR_NULL_PTR;
  size_t wo_off, total;
  const int rc = packed_plan(d, e, s, dtype, &wo_off, &total);
  if (rc != FLASHGAU_OK) return rc;
  *out_bytes = total;
  return FLASHGAU_OK;
}

int flashgau_pack_weights(const void* W_u, const void* W_v, const void* W_z, const void* W_o,
                          int64_t d, int64_t e, int64_t s, flashgau_dtype dtype, void* packed,
                          size_t packed_bytes, void* hip_stream) {
  size_t wo_off, total;
  const int rc = packed_plan(d, e, s, dtype, &wo_off, &total);
  if (rc != FLASHGAU_OK) return rc;
  if (!W_u || !W_v || !W_z || !W_o || !packed) return FLASHGAU_ERR_NULL_PTR;
  if (misaligned(W_u) || misaligned(W_v) || misaligned(W_z) || misaligned(W_o) || misaligned(packed))
    return FLASHGAU_ERR_MISALIGNED;
  if (packed_bytes < total) return FLASHGAU_ERR_WORKSPACE;
  const size_t esz = dtype == FLASHGAU_BF16 ? 2 : 4;
  const size_t nde = size_t(d) * size_t(e) * esz, nds = size_t(d) * size_t(s) * esz;
  if (overlaps(packed, total, W_u, nde) || overlaps(packed, total, W_v, nde) ||
      overlaps(packed, total, W_z, nds) || overlaps(packed, total, W_o, nde))
    return FLASHGAU_ERR_ALIASING;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  char* base = reinterpret_cast<char*>(packed);
  if (dtype == FLASHGAU_BF16)
    launch_pack<BF16>(W_u, W_v, W_z, W_o, int(d), int(e), int(s), reinterpret_cast<uint16_t*>(base),
                      reinterpret_cast<uint16_t*>(base + wo_off), stream);
  else
    launch_pack<F32>(W_u, W_v, W_z, W_o, int(d), int(e), int(s), reinterpret_cast<float*>(base),
                     reinterpret_cast<float*>(base + wo_off), stream);
  return hipGetLastError() == hipSuccess ? FLASHGAU_OK : FLASHGAU_ERR_HIP;
}

const char* flashgau_strerror(int code) {
  switch (code) {
    case FLASHGAU_OK: return "success";
    case FLASHGAU_ERR_NULL_PTR: return "a required pointer is NULL";
    case FLASHGAU_ERR_BAD_SHAPE:
      return "bad shape or argument (size < 1, n % chunk != 0, a size overflows, position or "
             "rotary base out of range)";
    case FLASHGAU_ERR_UNSUPPORTED:
      return "unsupported (dtype; d, e, s, chunk not a multiple of 8; or a chunk so long that the "
             "B*n*chunk score buffer exceeds 2^33 elements)";
    case FLASHGAU_ERR_MISALIGNED: return "a tensor pointer is not 16-byte aligned";
    case FLASHGAU_ERR_WORKSPACE: return "workspace smaller than flashgau_workspace_size()";
    case FLASHGAU_ERR_ALIASING: return "output or workspace overlaps an input or each other";
    case FLASHGAU_ERR_HIP: return "the HIP runtime rejected a kernel launch";
    case FLASHGAU_ERR_TOO_LARGE:
      return "the problem needs more workspace than flash_gau_forward_noalloc's fixed scratch holds";
    default: return "unknown error";
  }
}

}  // extern "C"
