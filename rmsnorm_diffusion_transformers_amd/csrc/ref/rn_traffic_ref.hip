// rn_traffic_ref.hip -- measurement references, not part of the operation.
//
// rn_traffic_ref: a kernel with the memory traffic of the fused residual + gate + LayerNorm +
// scale/shift op at D = 5120 with per-frame gate/scale/shift (sglang PR
// #36349, "Microbenchmark": operand order; sglang PR #33144,
// "Modifications": the (B, F, 1, C) layout) and none of its arithmetic:
//   residual_out = x ^ residual            (bitwise, per 16-byte vector)
//   y            = residual_out ^ gate ^ scale ^ shift
// with the fused kernel's geometry and memory instruction stream: one wave64
// per row, 4 rows per workgroup, 10 vectors of 16 bytes per lane; the
// frame's gate, scale and shift rows first (default cache policy, so they
// stay in L2), then x and residual (non-temporal, 8 cycles apart), at raised
// wave priority; then the residual_out stores and the y stores (non-
// temporal, 16 cycles apart).  Every byte of x, residual, residual_out and
// y crosses HBM once, as in the fused op.  The rate this kernel reaches on a
// placement of the four streams is what that traffic allows there without
// the statistics and the epilogue, the reference the fused kernel's rate is
// read against.
//
// rn_traffic_ref_nss: the same for the norm-only op at D = 5120 with
// broadcast (1, C) scale/shift: y = x ^ scale ^ shift, one wave64 per row, 2
// rows per workgroup, the scale and shift rows first (default policy), then x
// (non-temporal, back to back), at raised wave priority, then the y stores
// (non-temporal, 16 cycles apart) -- the norm-only kernel's stream for large
// problems.  Without arithmetic the kernel needs fewer registers; 40 KB of
// LDS per workgroup (unused) holds it to 4 workgroups per CU, i.e. 2 waves
// per SIMD, the norm-only kernel's occupancy.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kVpt = 10;
constexpr int kRowsPerBlock = 4;
constexpr int64_t kD = kWave * 8 * kVpt;  // 5120 bf16
constexpr uint32_t kRowBytes = (uint32_t)kD * 2u;
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;  // nt

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

template <int N>
__device__ __forceinline__ void spacing() {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("s_nop 7");
}

template <int POLICY, int N>
__device__ __forceinline__ u32x4 load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4 v = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POLICY));
  if constexpr (N > 0) spacing<N>();
  return v;
}

__device__ __forceinline__ void store(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kPolicyStream);
  spacing<2>();
}

struct RefArgs {
  void* y;
  void* residual_out;
  const void* x;
  const void* residual;
  const void* gate;
  const void* scale;
  const void* shift;
  uint32_t rows;
  uint32_t L;
  uint32_t frames;
  uint32_t tokens_per_frame;
};

__global__ __launch_bounds__(kWave * kRowsPerBlock) void traffic_ref_kernel(const RefArgs a) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t r = blockIdx.x * kRowsPerBlock + wave;
  if (r >= a.rows) return;
  const uint32_t b = r / a.L;
  const uint32_t frow = b * a.frames + (r - b * a.L) / a.tokens_per_frame;
  const uint64_t off = (uint64_t)r * kRowBytes;
  const uint64_t moff = (uint64_t)frow * kRowBytes;
  const uint32_t base = lane * 16u;
  u32x4 g[kVpt], s[kVpt], t[kVpt], x[kVpt], h[kVpt];
  __builtin_amdgcn_s_setprio(3);
  const auto rg = rsrc((const char*)a.gate + moff, kRowBytes);
  const auto rs = rsrc((const char*)a.scale + moff, kRowBytes);
  const auto rt = rsrc((const char*)a.shift + moff, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) g[v] = load<kPolicyDefault, 0>(rg, base + v * 1024u);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) s[v] = load<kPolicyDefault, 0>(rs, base + v * 1024u);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) t[v] = load<kPolicyDefault, 0>(rt, base + v * 1024u);
  const auto rx = rsrc((const char*)a.x + off, kRowBytes);
  const auto rr = rsrc((const char*)a.residual + off, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) x[v] = load<kPolicyStream, 1>(rx, base + v * 1024u);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) h[v] = load<kPolicyStream, 1>(rr, base + v * 1024u);
  __builtin_amdgcn_s_setprio(0);
  const auto ro = rsrc((char*)a.residual_out + off, kRowBytes);
  const auto ry = rsrc((char*)a.y + off, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) {
    h[v] ^= x[v];
    store(h[v], ro, base + v * 1024u);
  }
#pragma unroll
  for (int v = 0; v < kVpt; ++v) store(h[v] ^ g[v] ^ s[v] ^ t[v], ry, base + v * 1024u);
}

struct NssRefArgs {
  void* y;
  const void* x;
  const void* scale;
  const void* shift;
  uint32_t rows;
};

constexpr int kNssRowsPerBlock = 2;
constexpr size_t kNssLdsBytes = 40960;  // 4 workgroups in the 160 KB of a CU

__global__ __launch_bounds__(kWave * kNssRowsPerBlock) void traffic_ref_nss_kernel(const NssRefArgs a) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t r = blockIdx.x * kNssRowsPerBlock + wave;
  if (r >= a.rows) return;
  const uint64_t off = (uint64_t)r * kRowBytes;
  const uint32_t base = lane * 16u;
  u32x4 s[kVpt], t[kVpt], x[kVpt];
  __builtin_amdgcn_s_setprio(3);
  const auto rs = rsrc(a.scale, kRowBytes);
  const auto rt = rsrc(a.shift, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) s[v] = load<kPolicyDefault, 0>(rs, base + v * 1024u);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) t[v] = load<kPolicyDefault, 0>(rt, base + v * 1024u);
  const auto rx = rsrc((const char*)a.x + off, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) x[v] = load<kPolicyStream, 0>(rx, base + v * 1024u);
  __builtin_amdgcn_s_setprio(0);
  const auto ry = rsrc((char*)a.y + off, kRowBytes);
#pragma unroll
  for (int v = 0; v < kVpt; ++v) store(x[v] ^ s[v] ^ t[v], ry, base + v * 1024u);
}

}  // namespace

// Enqueue the reference on `stream`: [B, L, 5120] bf16 x, residual,
// residual_out and y (contiguous rows), gate/scale/shift of [B, frames,
// 5120] (frame-major rows; token l of batch b uses frame row
// b * frames + l / (L / frames)).  Device pointers.  Returns 0, or 1 for
// arguments it does not take (D other than 5120, L not a multiple of frames,
// more than 2^31 - 1 rows, a null pointer with rows), or 2 when the launch
// fails.  Nothing is launched for B * L = 0.
extern "C" int rn_traffic_ref(void* y, void* residual_out, const void* x, const void* residual,
                              const void* gate, const void* scale, const void* shift, int64_t B,
                              int64_t L, int64_t D, int64_t frames, hipStream_t stream) {
  if (D != kD || B < 0 || L < 0 || frames < 1 || L % frames != 0) return 1;
  const int64_t rows = B * L;
  if (rows == 0) return 0;
  if (rows > INT32_MAX || B * frames > INT32_MAX) return 1;
  if (!y || !residual_out || !x || !residual || !gate || !scale || !shift) return 1;
  RefArgs a{y, residual_out, x, residual, gate, scale, shift, (uint32_t)rows, (uint32_t)L,
            (uint32_t)frames, (uint32_t)(L / frames)};
  const dim3 grid((uint32_t)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(traffic_ref_kernel, grid, dim3(kWave * kRowsPerBlock), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Enqueue the norm-only reference on `stream`: [B, L, 5120] bf16 x and y
// (contiguous rows), broadcast scale and shift of 5120 bf16 each.  Device
// pointers.  Returns 0, 1 for arguments it does not take (D other than
// 5120, more than 2^31 - 1 rows, a null pointer with rows), or 2 when the
// launch fails.  Nothing is launched for B * L = 0.
extern "C" int rn_traffic_ref_nss(void* y, const void* x, const void* scale, const void* shift,
                                  int64_t B, int64_t L, int64_t D, hipStream_t stream) {
  if (D != kD || B < 0 || L < 0) return 1;
  const int64_t rows = B * L;
  if (rows == 0) return 0;
  if (rows > INT32_MAX) return 1;
  if (!y || !x || !scale || !shift) return 1;
  NssRefArgs a{y, x, scale, shift, (uint32_t)rows};
  const dim3 grid((uint32_t)((rows + kNssRowsPerBlock - 1) / kNssRowsPerBlock));
  hipLaunchKernelGGL(traffic_ref_nss_kernel, grid, dim3(kWave * kNssRowsPerBlock), kNssLdsBytes, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
