// probe.hip -- measured ceilings of one MI355X (gfx950) for the kernels of
// cce.hip: the bf16 MFMA rate under the chip's power limit, the LDS read
// bandwidth of a compute unit, and the rate at which all compute units can
// bring 16-byte-per-lane loads in (direct to LDS, as the GEMM loops do, or into
// registers) when the data sits in each XCD's L2 and when it does not.  These
// are the ceilings the roofline of the Cut Cross-Entropy kernels is read
// against; none of it is on the loss path.
//
// Every probe allocates and frees its own device buffers and synchronises;
// each returns 0 on success or the HIP error code.

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void *lds_ptr_t;

constexpr int NT = 512;  // 8 waves per workgroup, as the GEMM kernels run

// 16 independent accumulators of v_mfma_f32_16x16x32_bf16 per wave, each
// instruction reading register operands only.  Operands are pseudo-random
// bf16 in [-2, 2) (or zeros), a different pattern per lane.
__global__ __launch_bounds__(NT) void k_mfma(int iters, int zeros, float *out) {
  const uint32_t t = blockIdx.x * NT + threadIdx.x;
  u32x4 a[2], b[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t h = (t * 4 + e + i * 977) * 2654435761u;
      h ^= h >> 15;
      h *= 2246822519u;
      // two bf16: sign and exponent in [-2, 2), random mantissa
      const uint32_t lo = (h & 0x807fu) | 0x3f00u, hi = ((h >> 16) & 0x807fu) | 0x3f80u;
      a[i][e] = zeros ? 0u : (lo | (hi << 16));
      b[i][e] = zeros ? 0u : (hi | (lo << 16));
    }
  }
  f32x4 acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i & 1]),
                                                       __builtin_bit_cast(bf16x8, b[(i >> 1) & 1]),
                                                       acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  if (s == 1234.5f) out[t] = s;  // keeps the products live
}

// LDS reads: every thread reads 16 bytes per access; a 16-lane group reads
// 256 contiguous bytes (no bank conflicts); the address moves every
// iteration so nothing can be hoisted.  64 KiB per workgroup, so two
// workgroups (16 waves) share a compute unit.
__global__ __launch_bounds__(NT) void k_lds(int iters, uint32_t *out) {
  __shared__ __attribute__((aligned(16))) uint32_t s[16384];  // 64 KiB
  const int t = threadIdx.x;
  for (int i = t; i < 16384; i += NT) s[i] = (uint32_t)i * 2654435761u;
  __syncthreads();
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = (t * 4 + it * 1024 + j * 2048) & 16383;
      acc ^= *reinterpret_cast<const u32x4 *>(&s[idx]);
    }
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[blockIdx.x] = 1u;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, 0x00020000);
}

// Streaming loads: each workgroup walks a window of `win` bytes (its own, or
// one window shared by all) in 16 KiB steps, 8 waves x 2 loads of 1 KiB per
// step.  LDS: direct-to-LDS loads into a ring of 9 slots, 6 steps in flight
// (no LDS reader; the waves meet at a barrier every 4 steps).  Registers:
// 4 steps in flight, folded into a checksum.  Every offset is inside the
// window, and the window inside the buffer (host-checked).
__global__ __launch_bounds__(NT) void k_stream_lds(const uint8_t *src, int64_t win_stride, int win,
                                                   int iters, uint32_t *out) {
  __shared__ __attribute__((aligned(16))) uint8_t s[9 * 16384];
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src + (int64_t)blockIdx.x * win_stride, win);
  for (int it = 0; it < iters; ++it) {
    const int step = (int)(((int64_t)it * 16384) % win);
    uint8_t *slot = s + (it % 9) * 16384;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(slot + (w * 2 + j) * 1024), 16,
                                               step + (w * 2 + j) * 1024 + l * 16, 0, 0, 0);
    __builtin_amdgcn_s_waitcnt((10 & 15) | 0x0070);  // vmcnt(10): 6 steps in flight
    if ((it & 3) == 3) __builtin_amdgcn_s_barrier();
  }
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  if (s[t * 7] == 0xab && s[t * 13] == 0xcd) out[blockIdx.x] = 1u;
}

__global__ __launch_bounds__(NT) void k_stream_reg(const uint8_t *src, int64_t win_stride, int win,
                                                   int iters, uint32_t *out) {
  const int t = threadIdx.x, l = t & 63, w = t >> 6;
  const __amdgpu_buffer_rsrc_t rs = rsrc(src + (int64_t)blockIdx.x * win_stride, win);
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 r[4][2];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int j = 0; j < 2; ++j) r[d][j] = u32x4{0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int step = (int)(((int64_t)(it + d) * 16384) % win);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        acc ^= r[d][j];
        r[d][j] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, step + (w * 2 + j) * 1024 + l * 16, 0, 0));
      }
    }
  }
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc ^= r[d][j];
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[blockIdx.x] = 1u;
}

int cus_of_device() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cus;
}

// Times `launch` (already warmed) between two events on the null stream.
template <typename F>
hipError_t timed(F launch, float *ms) {
  hipEvent_t a, b;
  hipError_t e = hipEventCreate(&a);
  if (e != hipSuccess) return e;
  if ((e = hipEventCreate(&b)) != hipSuccess) return e;
  launch();
  if ((e = hipEventRecord(a, 0)) == hipSuccess) {
    launch();
    if ((e = hipGetLastError()) == hipSuccess && (e = hipEventRecord(b, 0)) == hipSuccess &&
        (e = hipEventSynchronize(b)) == hipSuccess)
      e = hipEventElapsedTime(ms, a, b);
  }
  hipEventDestroy(a);
  hipEventDestroy(b);
  return e;
}

}  // namespace

extern "C" {

// bf16 MFMA throughput: *flops over *ms.  zeros != 0 runs the same
// instructions on zero operands (the power the operands' bits cost).
int cce_probe_mfma(int zeros, float *ms, double *flops) {
  const int cus = cus_of_device();
  if (cus <= 0) return (int)hipErrorInvalidDevice;
  float *out = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)cus * 2 * NT * sizeof(float));
  if (e != hipSuccess) return (int)e;
  const int iters = 60000, grid = cus * 2;
  e = timed([&] { k_mfma<<<grid, NT>>>(iters, zeros, out); }, ms);
  *flops = (double)grid * (NT / 64) * iters * 16 * (16.0 * 16 * 32 * 2);
  hipFree(out);
  return (int)e;
}

// LDS read bandwidth of all compute units: *bytes over *ms.
int cce_probe_lds(float *ms, double *bytes) {
  const int cus = cus_of_device();
  if (cus <= 0) return (int)hipErrorInvalidDevice;
  uint32_t *out = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)cus * 2 * 4);
  if (e != hipSuccess) return (int)e;
  const int iters = 4000, grid = 2 * cus;
  e = timed([&] { k_lds<<<grid, NT>>>(iters, out); }, ms);
  *bytes = (double)grid * NT * 16 * 8 * iters;
  hipFree(out);
  return (int)e;
}

// Streaming loads by one workgroup per compute unit over windows of
// window_bytes (a multiple of 16 KiB, at most 16 MiB): shared != 0 gives
// every workgroup the same window, else each its own (consecutive windows);
// to_lds selects direct-to-LDS loads, else loads into registers.
int cce_probe_stream(int64_t window_bytes, int shared, int to_lds, float *ms, double *bytes) {
  const int cus = cus_of_device();
  if (cus <= 0) return (int)hipErrorInvalidDevice;
  if (window_bytes < 16384 || window_bytes > (16 << 20) || window_bytes % 16384)
    return (int)hipErrorInvalidValue;
  const int64_t stride = shared ? 0 : window_bytes;
  const size_t total = (size_t)(shared ? window_bytes : window_bytes * cus);
  uint8_t *src = nullptr;
  uint32_t *out = nullptr;
  hipError_t e = hipMalloc(&src, total);
  if (e != hipSuccess) return (int)e;
  if ((e = hipMalloc(&out, (size_t)cus * 4)) != hipSuccess) {
    hipFree(src);
    return (int)e;
  }
  if ((e = hipMemset(src, 1, total)) == hipSuccess) {
    const int iters = 16000, win = (int)window_bytes;
    if (to_lds)
      e = timed([&] { k_stream_lds<<<cus, NT>>>(src, stride, win, iters, out); }, ms);
    else
      e = timed([&] { k_stream_reg<<<cus, NT>>>(src, stride, win, iters, out); }, ms);
    *bytes = (double)cus * 16384 * iters;
  }
  hipFree(out);
  hipFree(src);
  return (int)e;
}

}  // extern "C"
