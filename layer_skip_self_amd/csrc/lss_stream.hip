// Streaming-read ceiling of the decode projections on this GPU: read the
// bytes of one weight matrix (N rows x K bf16) and only reduce them, with the
// decode GEMV's access pattern or a fully contiguous walk, timed with HIP
// events.  Eight distinct matrices are read round robin, so no launch finds
// its bytes in the last-level cache (256 MB on MI355X).  The rate of such a
// load-only kernel is the achievable ceiling below the 8 TB/s HBM peak that
// a GEMV of the same shape and launch can approach.
//
//   lss_stream N K [workgroups ...]   (default 256, 512 and 1024 workgroups)
//
// Patterns (one 512-thread workgroup = 8 waves; lane l of a wave loads the
// 16 bytes at offset 16 l of a 1 KB piece, nontemporal):
//   rows:   the GEMV's: workgroup g takes a contiguous range of rows, in
//           groups of 8; wave w takes the 1 KB pieces w, w + 8, w + 16, ...
//           of the P pieces of a row, and reads each piece of the group's 8
//           rows in one step (8 loads);
//   ranges: as rows, but wave w takes the contiguous pieces
//           [w P / 8, (w + 1) P / 8);
//   contig: workgroup g takes a contiguous byte range; each wave step reads
//           16 consecutive 1 KB pieces.
// Every case is bounds-checked on the host (the ranges cover the matrix
// exactly or are clamped to its last piece).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <vector>

namespace {

#define SCHK(x)                                                                        \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

// rows / ranges patterns: rows [g * rpw, (g + 1) * rpw) of N, 8 rows per step
__global__ __launch_bounds__(512) void k_read_rows(const u32x4* __restrict__ w, int N, int pieces, int rpw,
                                                   int ranges, unsigned* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r0 = blockIdx.x * rpw, r1 = min(N, r0 + rpw);
  unsigned acc = 0;
  const int c0 = ranges ? wave * pieces / 8 : wave, c1 = ranges ? (wave + 1) * pieces / 8 : pieces;
  const int cs = ranges ? 1 : 8;
  for (int t = r0; t < r1; t += 8)
    for (int c = c0; c < c1; c += cs) {
      u32x4 v[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const size_t row = (size_t)min(t + r, N - 1);
        v[r] = ld_nt(w + (row * pieces + c) * 64 + lane);
      }
#pragma unroll
      for (int r = 0; r < 8; ++r) acc += v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
    }
  out[blockIdx.x * 512 + threadIdx.x] = acc;
}

// contiguous pattern: pieces [g * ppw, (g + 1) * ppw) of the matrix
__global__ __launch_bounds__(512) void k_read_contig(const u32x4* __restrict__ w, long total, long ppw,
                                                     unsigned* __restrict__ out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long p0 = (long)blockIdx.x * ppw, p1 = p0 + ppw < total ? p0 + ppw : total;
  unsigned acc = 0;
  for (long s = p0 + 16L * wave; s < p1; s += 128) {
    u32x4 v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const long pc = s + r < total ? s + r : total - 1;
      v[r] = ld_nt(w + pc * 64 + lane);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) acc += v[r].x ^ v[r].y ^ v[r].z ^ v[r].w;
  }
  out[blockIdx.x * 512 + threadIdx.x] = acc;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 3) {
    std::fprintf(stderr, "usage: %s N K [workgroups ...]\n", argv[0]);
    return 2;
  }
  const int N = std::atoi(argv[1]), K = std::atoi(argv[2]);
  if (N < 8 || K < 512 || K % 512 != 0) {
    std::fprintf(stderr, "N >= 8 and K a multiple of 512 (1 KB rows of bf16 pieces)\n");
    return 2;
  }
  std::vector<int> wgs;
  for (int i = 3; i < argc; ++i) wgs.push_back(std::atoi(argv[i]));
  if (wgs.empty()) wgs = {256, 512, 1024};
  const int pieces = K / 512;                      // 1 KB pieces per row
  const size_t bytes = (size_t)N * K * 2;
  const long total = (long)N * pieces;
  const int NB = 8, REPS = 64;
  std::vector<u32x4*> buf(NB);
  for (auto& b : buf) {
    SCHK(hipMalloc(&b, bytes));
    SCHK(hipMemset(b, 1, bytes));
  }
  int maxwg = 0;
  for (int g : wgs) maxwg = g > maxwg ? g : maxwg;
  if (maxwg < 1 || maxwg > 65536) {
    std::fprintf(stderr, "workgroups must be in 1 .. 65536\n");
    return 2;
  }
  unsigned* out;
  SCHK(hipMalloc(&out, (size_t)maxwg * 512 * sizeof(unsigned)));
  hipEvent_t e0, e1;
  SCHK(hipEventCreate(&e0));
  SCHK(hipEventCreate(&e1));
  auto run = [&](int pat, int wg) -> double {   // 0 rows, 1 ranges, 2 contig
    const int rpw = ((N + wg - 1) / wg + 7) / 8 * 8;        // rows per workgroup, whole groups of 8
    const long ppw = (total + wg - 1) / wg;
    auto launch = [&](int i) {
      if (pat < 2)
        hipLaunchKernelGGL(k_read_rows, dim3(wg), dim3(512), 0, 0, buf[i % NB], N, pieces, rpw, pat, out);
      else
        hipLaunchKernelGGL(k_read_contig, dim3(wg), dim3(512), 0, 0, buf[i % NB], total, ppw, out);
    };
    for (int i = 0; i < NB; ++i) launch(i);
    SCHK(hipEventRecord(e0));
    for (int i = 0; i < REPS; ++i) launch(i);
    SCHK(hipEventRecord(e1));
    SCHK(hipEventSynchronize(e1));
    SCHK(hipGetLastError());
    float ms = 0.f;
    SCHK(hipEventElapsedTime(&ms, e0, e1));
    return 1e3 * ms / REPS;
  };
  for (int pass = 0; pass < 2; ++pass)
    for (int wg : wgs)
      for (int pat = 0; pat < 3; ++pat) {
        const double us = run(pat, wg);
        if (pass == 1)
          std::printf("{\"N\": %d, \"K\": %d, \"MB\": %.2f, \"pattern\": \"%s\", \"workgroups\": %d, \"us\": %.2f, "
                      "\"GBps\": %.0f, \"frac_of_8TBps\": %.3f}\n",
                      N, K, bytes / 1e6, pat == 0 ? "rows" : pat == 1 ? "ranges" : "contig", wg, us,
                      bytes / (us * 1e-6) / 1e9,
                      bytes / (us * 1e-6) / 8e12);
      }
  for (auto& b : buf) SCHK(hipFree(b));
  SCHK(hipFree(out));
  return 0;
}
