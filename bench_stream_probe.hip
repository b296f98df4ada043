// Read-bandwidth ceiling of the batched decode's launch shapes on one GPU: the bytes a
// 256-sequence x 4-KV-head decode streams (a 128-slot ring of 32 KB of K and 32 KB of V
// per (sequence, KV head), 64 MiB in all), read once by kernels that do nothing with the
// data but fold it into 16 bytes per thread, in several workgroup shapes: one
// workgroup per ring with 128 / 256 / 512 threads, a ring split over 2 / 4 / 8
// workgroups, and one wavefront per ring streaming it in chunks; the one-workgroup and
// split shapes also with the loads marked non-temporal (as the decode's bf16 ring loads
// are).  The FP8 ring's shape (16 KB of K codes + 16 KB of V codes per ring, 32 MiB in
// all) is read by one 256-thread workgroup per ring, with 16-byte loads and with the V
// codes as 8-byte loads (as the FP8 decode reads them); a launch that reads nothing and
// writes the same 16 bytes per thread gives the floor of a 1024-workgroup launch.  32
// input sets (2 GiB) are rotated so that no launch finds its data in the 256 MB
// Infinity Cache.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/bench_stream_probe bench_stream_probe.hip
//   /tmp/bench_stream_probe
//
// Prints the average time per launch (HIP events over 400 launches) and GB/s.
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <vector>

#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("%s failed: %s\n", #x, hipGetErrorString(e)); return 1; } } while (0)

constexpr int kRings = 1024;         // 256 x 4
constexpr int kUnits = 2048;         // 16-byte units per ring per tensor (32 KB)

template <bool NT>
__device__ __forceinline__ uint4 load16(const uint4* p) {
  if constexpr (NT) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}

template <int THREADS, int SPLIT, bool NT = false, int UNITS = kUnits>
__global__ __launch_bounds__(THREADS) void stream_k(const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                     uint4* __restrict__ out) {
  constexpr int PER = UNITS / SPLIT / THREADS;  // units per thread per tensor
  const int ring = blockIdx.x / SPLIT, part = blockIdx.x % SPLIT;
  const uint4* kb = K + (size_t)ring * UNITS + part * (UNITS / SPLIT);
  const uint4* vb = V + (size_t)ring * UNITS + part * (UNITS / SPLIT);
  uint4 r[2 * PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) r[j] = load16<NT>(kb + j * THREADS + threadIdx.x);
#pragma unroll
  for (int j = 0; j < PER; ++j) r[PER + j] = load16<NT>(vb + j * THREADS + threadIdx.x);
  uint4 acc = r[0];
#pragma unroll
  for (int j = 1; j < 2 * PER; ++j) { acc.x ^= r[j].x; acc.y += r[j].y; acc.z ^= r[j].z; acc.w += r[j].w; }
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = acc;
}

// FP8-ring shape: 1024 16-byte units of K codes per ring read 16 bytes at a time, the V
// codes 8 bytes at a time (2048 8-byte pieces per ring)
template <int THREADS>
__global__ __launch_bounds__(THREADS) void stream_fp8v8(const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                         uint4* __restrict__ out) {
  constexpr int UNITS = kUnits / 2, PK = UNITS / THREADS, PV = 2 * UNITS / THREADS;
  const uint4* kb = K + (size_t)blockIdx.x * UNITS;
  const uint2* vb = reinterpret_cast<const uint2*>(V + (size_t)blockIdx.x * UNITS);
  uint4 r[PK];
  uint2 q[PV];
#pragma unroll
  for (int j = 0; j < PK; ++j) r[j] = kb[j * THREADS + threadIdx.x];
#pragma unroll
  for (int j = 0; j < PV; ++j) q[j] = vb[j * THREADS + threadIdx.x];
  uint4 acc = r[0];
#pragma unroll
  for (int j = 1; j < PK; ++j) { acc.x ^= r[j].x; acc.y += r[j].y; acc.z ^= r[j].z; acc.w += r[j].w; }
#pragma unroll
  for (int j = 0; j < PV; ++j) { acc.x ^= q[j].x; acc.y += q[j].y; }
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = acc;
}

// the same launch shape with no reads
template <int THREADS>
__global__ __launch_bounds__(THREADS) void write_only(uint4* __restrict__ out, unsigned seed) {
  out[(size_t)blockIdx.x * THREADS + threadIdx.x] = make_uint4(seed, blockIdx.x, threadIdx.x, 0u);
}

// one wavefront per ring, loads issued in chunks of C units per lane in flight
template <int C>
__global__ __launch_bounds__(64) void stream_wave(const uint4* __restrict__ K, const uint4* __restrict__ V,
                                                  uint4* __restrict__ out) {
  const int ring = blockIdx.x;
  const uint4* kb = K + (size_t)ring * kUnits;
  const uint4* vb = V + (size_t)ring * kUnits;
  uint4 acc = {0, 0, 0, 0};
  for (int c0 = 0; c0 < 2 * kUnits / 64; c0 += C) {
    uint4 r[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
      const int u = (c0 + j) * 64 + threadIdx.x;
      r[j] = u < kUnits ? kb[u] : vb[u - kUnits];
    }
#pragma unroll
    for (int j = 0; j < C; ++j) { acc.x ^= r[j].x; acc.y += r[j].y; acc.z ^= r[j].z; acc.w += r[j].w; }
  }
  out[(size_t)blockIdx.x * 64 + threadIdx.x] = acc;
}

__global__ void fill(uint4* p, size_t n, unsigned seed) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4((unsigned)i * 2654435761u ^ seed, (unsigned)i, seed, (unsigned)(i >> 7));
}

constexpr int kSets = 32;

template <typename F>
float time_it(F launch, int iters) {
  hipEvent_t a, b;
  (void)hipEventCreate(&a);
  (void)hipEventCreate(&b);
  for (int i = 0; i < 64; ++i) launch(i % kSets);
  (void)hipDeviceSynchronize();
  (void)hipEventRecord(a, 0);
  for (int i = 0; i < iters; ++i) launch(i % kSets);
  (void)hipEventRecord(b, 0);
  (void)hipEventSynchronize(b);
  float ms = 0.f;
  (void)hipEventElapsedTime(&ms, a, b);
  return ms * 1000.f / iters;
}

int main() {
  const size_t units = (size_t)kRings * kUnits;  // per tensor per set
  std::vector<uint4*> K(kSets), V(kSets);
  for (int s = 0; s < kSets; ++s) {
    CHECK(hipMalloc(&K[s], units * 16));
    CHECK(hipMalloc(&V[s], units * 16));
    fill<<<1024, 256>>>(K[s], units, 2 * s);
    fill<<<1024, 256>>>(V[s], units, 2 * s + 1);
  }
  uint4* out;
  CHECK(hipMalloc(&out, (size_t)64 << 20));
  CHECK(hipDeviceSynchronize());
  const double bytes = 2.0 * units * 16;
  const int iters = 400;
#define RUN(T, S)                                                                                  \
  {                                                                                                \
    float us = time_it([&](int s) { stream_k<T, S><<<kRings * S, T>>>(K[s], V[s], out); }, iters); \
    printf("stream threads=%4d split=%d  wgs=%5d  bytes/wg=%6d  %7.2f us  %6.0f GB/s\n", T, S,      \
           kRings * S, 65536 / S, us, bytes / us / 1e3);                                           \
  }
  RUN(256, 1) RUN(512, 1) RUN(128, 1) RUN(256, 2) RUN(128, 2) RUN(64, 4) RUN(128, 4) RUN(256, 4)
  RUN(64, 8) RUN(256, 8) RUN(64, 2)
#define RUNNT(T, S)                                                                                     \
  {                                                                                                     \
    float us = time_it([&](int s) { stream_k<T, S, true><<<kRings * S, T>>>(K[s], V[s], out); }, iters); \
    printf("stream-nt threads=%4d split=%d  wgs=%5d  bytes/wg=%6d  %7.2f us  %6.0f GB/s\n", T, S,        \
           kRings * S, 65536 / S, us, bytes / us / 1e3);                                                \
  }
  RUNNT(256, 1) RUNNT(128, 1) RUNNT(128, 2) RUNNT(64, 2) RUNNT(64, 4)
#define RUNW(C)                                                                                   \
  {                                                                                               \
    float us = time_it([&](int s) { stream_wave<C><<<kRings, 64>>>(K[s], V[s], out); }, iters);    \
    printf("wave-per-ring chunk=%2d  %7.2f us  %6.0f GB/s\n", C, us, bytes / us / 1e3);             \
  }
  RUNW(8) RUNW(16) RUNW(32)
  {
    const double b8 = bytes / 2;
    float us = time_it([&](int s) { stream_k<256, 1, false, kUnits / 2><<<kRings, 256>>>(K[s], V[s], out); }, iters);
    printf("fp8-ring threads= 256 16-byte loads        %7.2f us  %6.0f GB/s\n", us, b8 / us / 1e3);
    us = time_it([&](int s) { stream_k<256, 1, true, kUnits / 2><<<kRings, 256>>>(K[s], V[s], out); }, iters);
    printf("fp8-ring threads= 256 16-byte loads, nt    %7.2f us  %6.0f GB/s\n", us, b8 / us / 1e3);
    us = time_it([&](int s) { stream_fp8v8<256><<<kRings, 256>>>(K[s], V[s], out); }, iters);
    printf("fp8-ring threads= 256 K 16-byte, V 8-byte  %7.2f us  %6.0f GB/s\n", us, b8 / us / 1e3);
    us = time_it([&](int s) { write_only<256><<<kRings, 256>>>(out, (unsigned)s); }, iters);
    printf("no reads threads= 256 wgs=1024             %7.2f us\n", us);
  }
  CHECK(hipDeviceSynchronize());
  printf("done\n");
  return 0;
}
