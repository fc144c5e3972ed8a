// HBM bandwidth probe (a measurement tool, not part of libcgtp): what the
// memory system sustains, with no arithmetic, for plain streaming writes and
// reads and for the row-segment patterns of the tensor product - 1,048,576
// rows; forward mix = read 26,240 B + write 79,872 B per row, backward mix =
// read 79,872 B + write 26,240 B per row, four row segments like the
// per-x-block launches. Built by build.py as clebsch_gordan_tensor_amd/hbm_probe.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdint>
#define CK(x) do { hipError_t e = (x); if (e != hipSuccess) { printf("HIP error %s at %d\n", hipGetErrorString(e), __LINE__); return 1; } } while (0)
typedef float f4 __attribute__((ext_vector_type(4)));

// (a) grid-stride float4 writes over n4 vectors
__global__ void k_fill(f4* p, int64_t n4) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) p[i] = f4{1.f, 2.f, 3.f, 4.f};
}
// (b) rows of R floats; group of LPR lanes per row, 4 floats per lane per store; rows per launch = B
// writes segment [seg_off, seg_off + seg_len) of every row
__global__ void k_rows(float* out, int64_t B, int R, int seg_off, int seg_len, int lpr_log2) {
  const int64_t gt = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t row = gt >> lpr_log2;
  const int lane = gt & ((1 << lpr_log2) - 1);
  if (row >= B) return;
  float* r = out + row * R + seg_off;
  const int step = (1 << lpr_log2) * 4;
  for (int c = lane * 4; c < seg_len; c += step) *(f4*)(r + c) = f4{1.f, 2.f, 3.f, (float)c};
}
// (c) rows with reads: read rd_len floats from in-row, write seg_len floats (like the forward's 1:3 mix)
__global__ void k_rows_rw(const float* in, float* out, int64_t B, int RI, int R, int rd_len, int seg_len, int lpr_log2) {
  const int64_t gt = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t row = gt >> lpr_log2;
  const int lane = gt & ((1 << lpr_log2) - 1);
  if (row >= B) return;
  const float* ri = in + row * RI;
  float* r = out + row * R;
  const int step = (1 << lpr_log2) * 4;
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  for (int c = lane * 4; c < rd_len; c += step) acc += *(const f4*)(ri + c);
  for (int c = lane * 4; c < seg_len; c += step) *(f4*)(r + c) = acc;
}
// (d) grid-stride float4 reads; one float per thread written
__global__ void k_read(const f4* p, int64_t n4, float* sink) {
  f4 acc = f4{0.f, 0.f, 0.f, 0.f};
  const int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t i = t; i < n4; i += (int64_t)gridDim.x * blockDim.x) acc += p[i];
  sink[t] = acc.x + acc.y + acc.z + acc.w;
}
int main() {
  const int64_t B = 1 << 20; const int R = 19968; const int RI = 6560;  // floats per row (out, in)
  float *out, *in;
  CK(hipMalloc(&out, (size_t)B * R * 4)); CK(hipMalloc(&in, (size_t)B * RI * 4));
  hipEvent_t a, b; CK(hipEventCreate(&a)); CK(hipEventCreate(&b)); float ms;
  const size_t bytes = (size_t)B * R * 4;
  // (a)
  k_fill<<<8192, 256>>>((f4*)out, (int64_t)B * R / 4); CK(hipDeviceSynchronize());
  CK(hipEventRecord(a)); for (int i = 0; i < 3; ++i) k_fill<<<8192, 256>>>((f4*)out, (int64_t)B * R / 4); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
  CK(hipEventElapsedTime(&ms, a, b)); printf("fill grid-stride          : %.2f TB/s\n", 3.0 * bytes / (ms * 1e-3) / 1e12);
  for (int lg = 4; lg <= 6; ++lg) {
    const int64_t threads = B << lg; const unsigned grid = (unsigned)((threads + 255) / 256);
    k_rows<<<grid, 256>>>(out, B, R, 0, R, lg); CK(hipDeviceSynchronize());
    CK(hipEventRecord(a)); for (int i = 0; i < 3; ++i) k_rows<<<grid, 256>>>(out, B, R, 0, R, lg); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b)); printf("rows whole (lanes/row %2d): %.2f TB/s\n", 1 << lg, 3.0 * bytes / (ms * 1e-3) / 1e12);
    // segments like the per-block launches: 4 segments of the row
    const int segs[5] = {0, 2048, 2048 + 4992, 2048 + 4992 + 6528, R};
    CK(hipEventRecord(a));
    for (int s = 0; s < 4; ++s) k_rows<<<grid, 256>>>(out, B, R, segs[s], segs[s + 1] - segs[s], lg);
    CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b)); printf("rows in 4 segments (%2d)  : %.2f TB/s\n", 1 << lg, 1.0 * bytes / (ms * 1e-3) / 1e12);
    CK(hipEventRecord(a)); for (int i = 0; i < 3; ++i) k_rows_rw<<<grid, 256>>>(in, out, B, RI, R, RI, R, lg); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b)); printf("rows read 26K + write 80K (%2d): %.2f TB/s\n", 1 << lg, 3.0 * (bytes + (size_t)B * RI * 4) / (ms * 1e-3) / 1e12);
  }
  {
    float* sink; CK(hipMalloc(&sink, 8192 * 256 * 4));
    k_read<<<8192, 256>>>((const f4*)out, (int64_t)B * R / 4, sink); CK(hipDeviceSynchronize());
    CK(hipEventRecord(a)); for (int i = 0; i < 3; ++i) k_read<<<8192, 256>>>((const f4*)out, (int64_t)B * R / 4, sink); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
    CK(hipEventElapsedTime(&ms, a, b)); printf("read grid-stride          : %.2f TB/s\n", 3.0 * bytes / (ms * 1e-3) / 1e12);
    // backward-like mix: read 26560 floats per row (from 'out' as a wider input), write 6560 floats (into 'in')
    const int RR = 19968, RW = 6560;
    for (int lg = 5; lg <= 6; ++lg) {
      const int64_t threads = B << lg; const unsigned grid = (unsigned)((threads + 255) / 256);
      k_rows_rw<<<grid, 256>>>(out, in, B, RR, RW, RR, RW, lg); CK(hipDeviceSynchronize());
      CK(hipEventRecord(a)); for (int i = 0; i < 3; ++i) k_rows_rw<<<grid, 256>>>(out, in, B, RR, RW, RR, RW, lg); CK(hipEventRecord(b)); CK(hipEventSynchronize(b));
      CK(hipEventElapsedTime(&ms, a, b)); printf("rows read 80K + write 26K (%2d): %.2f TB/s\n", 1 << lg, 3.0 * ((size_t)B * (RR + RW) * 4) / (ms * 1e-3) / 1e12);
    }
  }
  return 0;
}
