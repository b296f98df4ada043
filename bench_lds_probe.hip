// LDS read bandwidth of one compute unit on gfx950, as the attention kernels read LDS:
// 16-byte row reads (ds_read_b128) and 8-byte transposed reads (ds_read_b64_tr_b16), with
// 4, 8 or 16 wavefronts per workgroup and one workgroup per CU.  Every lane reads
// distinct consecutive 16-byte (8-byte) slots, so no access has a bank conflict; each
// wavefront times its own loop with the shader clock (s_memtime) and the CU's bytes per
// clock are the bytes all its wavefronts read over the longest wavefront's cycles.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//     -o /tmp/bench_lds_probe bench_lds_probe.hip
//   /tmp/bench_lds_probe
#include <hip/hip_runtime.h>
#include <stdio.h>

#include <vector>

#define CHECK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("%s failed: %s\n", #x, hipGetErrorString(e)); return 1; } } while (0)

constexpr int kIters = 4096;
constexpr int kLds = 64 * 1024;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int MODE>  // 0: ds_read_b128, 1: ds_read_b64_tr_b16
__global__ void lds_read(unsigned long long* cycles, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) char lds[kLds];
  for (int x = threadIdx.x; x < kLds / 4; x += blockDim.x) reinterpret_cast<unsigned*>(lds)[x] = x * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // each wavefront walks the whole LDS from its own starting point, one 1 KB (512-byte)
  // contiguous row of lanes per read, 8 reads per turn; the sums keep every read live
  const int base = w * 4096;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int row = (it * 8 + r) & 63;
      if constexpr (MODE == 0) {
        const int off = (base + row * 1024 + 16 * lane) & (kLds - 1);
        acc += *reinterpret_cast<const u32x4*>(lds + off);
      } else {
        const int off = (base + row * 1024 + 8 * lane) & (kLds - 1);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
        const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds + off));
        acc[r & 3] += (unsigned)(unsigned short)v[0] + ((unsigned)(unsigned short)v[1] << 16);
        acc[(r + 1) & 3] += (unsigned)(unsigned short)v[2] + ((unsigned)(unsigned short)v[3] << 16);
      }
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cycles[blockIdx.x * 16 + w] = t1 - t0;
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

template <int MODE>
int run(int waves, int nblocks) {
  unsigned long long* cyc;
  unsigned* sink;
  CHECK(hipMalloc(&cyc, (size_t)nblocks * 16 * 8));
  CHECK(hipMalloc(&sink, (size_t)nblocks * 1024 * 4));
  CHECK(hipMemset(cyc, 0, (size_t)nblocks * 16 * 8));
  lds_read<MODE><<<nblocks, waves * 64>>>(cyc, sink);  // warm-up
  CHECK(hipDeviceSynchronize());
  lds_read<MODE><<<nblocks, waves * 64>>>(cyc, sink);
  CHECK(hipDeviceSynchronize());
  std::vector<unsigned long long> h((size_t)nblocks * 16);
  CHECK(hipMemcpy(h.data(), cyc, h.size() * 8, hipMemcpyDeviceToHost));
  double sum_bpc = 0.0;
  for (int b = 0; b < nblocks; ++b) {
    unsigned long long mx = 0;
    for (int w = 0; w < waves; ++w) mx = h[(size_t)b * 16 + w] > mx ? h[(size_t)b * 16 + w] : mx;
    const double bytes = (double)waves * 64 * kIters * 8 * (MODE == 0 ? 16 : 8);
    sum_bpc += bytes / (double)mx;
  }
  printf("%s  wavefronts per CU %2d  %6.1f bytes per shader clock per CU (mean over %d CUs)\n",
         MODE == 0 ? "ds_read_b128     " : "ds_read_b64_tr_b16", waves, sum_bpc / nblocks, nblocks);
  CHECK(hipFree(cyc));
  CHECK(hipFree(sink));
  return 0;
}

int main() {
  int cus = 0;
  CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
  for (int waves : {4, 8, 16}) {
    if (run<0>(waves, cus)) return 1;
    if (run<1>(waves, cus)) return 1;
  }
  printf("done\n");
  return 0;
}
