// Graph preparation: COO -> CSR by destination, validation, and the
// source-ordered transpose used to sum grad_x without atomics.
//
// Receiver-ordered (CSR) aggregation without atomics and determinism are the
// design points of "E3J: An Efficient and Open-Source Backend for Euclidean
// Equivariant Operations on GPU and TPU", sections 1, C.2, E.2.2 and E.3.
// Here the integer layout is bit-exact and independent of thread timing:
// positions are first claimed with integer atomics (whose final counts are
// exact), then every segment is ordered by a unique key - (src, input index)
// for the CSR, the CSR position for the transpose. Segments are sorted in
// runs of kRun elements (each element's rank is the count of smaller keys in
// its run), then runs are merged pairwise until the longest segment is one
// run (each element's place in the merged run is its index in its own run
// plus the count of smaller keys in the partner run, by binary search). With
// unique keys every step has one result, and the cost is
// O(E (kRun + log^2 max degree)): a padding node receiving most of the edges
// (one segment of any length) costs no more than ordinary receivers.
#include <algorithm>
#include <memory>
#include <utility>
#include <vector>

#include "graph.hpp"

// Receiver schedule for the convolution kernels: a breadth-first order over
// the CSR (the neighbours of a receiver are its sources), components taken in
// index order. Receivers that are close in this order share many sources, so
// kernels that walk it (each XCD one contiguous range) read a source row into
// L2 once for several receivers. Results do not depend on the schedule: every
// receiver is summed by one owner in CSR order.
static std::vector<int32_t> receiver_schedule(int64_t N, const std::vector<int32_t>& row_ptr,
                                              const std::vector<int32_t>& src) {
  std::vector<int32_t> order;
  order.reserve(size_t(N));
  std::vector<char> seen(size_t(N), 0);
  for (int64_t start = 0; start < N; ++start) {
    if (seen[size_t(start)]) continue;
    seen[size_t(start)] = 1;
    size_t head = order.size();
    order.push_back(int32_t(start));
    while (head < order.size()) {
      const int32_t u = order[head++];
      for (int32_t e = row_ptr[size_t(u)]; e < row_ptr[size_t(u) + 1]; ++e) {
        const int32_t v = src[size_t(e)];
        if (!seen[size_t(v)]) {
          seen[size_t(v)] = 1;
          order.push_back(v);
        }
      }
    }
  }
  return order;
}

namespace cgtp {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 4;
constexpr int kScanTile = kScanThreads * kScanItems;

__global__ __launch_bounds__(kScanThreads) void scan_tiles(const int32_t* __restrict__ in,
                                                           int32_t* __restrict__ out,
                                                           int32_t* __restrict__ tile_sum, int64_t n) {
  __shared__ int32_t s[kScanThreads];
  const int tid = threadIdx.x;
  const int64_t base = int64_t(blockIdx.x) * kScanTile + int64_t(tid) * kScanItems;
  int32_t v[kScanItems];
  int32_t t = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    v[k] = base + k < n ? in[base + k] : 0;
    t += v[k];
  }
  s[tid] = t;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int32_t add = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += add;
    __syncthreads();
  }
  int32_t run = s[tid] - t;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    if (base + k < n) out[base + k] = run;
    run += v[k];
  }
  if (tid == kScanThreads - 1) tile_sum[blockIdx.x] = s[tid];
}

__global__ void scan_add(int32_t* __restrict__ out, const int32_t* __restrict__ tile_off, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) out[i] += tile_off[i / kScanTile];
}

__global__ void scan_total(int32_t* __restrict__ out, const int32_t* __restrict__ counts, int64_t n) {
  out[n] = n > 0 ? out[n - 1] + counts[n - 1] : 0;
}

struct DevBuf {
  void* p = nullptr;
  explicit DevBuf(size_t bytes) {
    if (bytes) CGTP_CHECK_HIP(hipMalloc(&p, bytes));
  }
  ~DevBuf() { (void)hipFree(p); }
  DevBuf(const DevBuf&) = delete;
  DevBuf& operator=(const DevBuf&) = delete;
  template <typename T>
  T* as() const {
    return static_cast<T*>(p);
  }
};

unsigned blocks_for(int64_t n, int threads) { return unsigned((n + threads - 1) / threads); }

// ---- CSR by destination
// flag[0]: invalid index seen; flag[1]: largest destination degree
__global__ void coo_count(const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                          int32_t* __restrict__ counts, int32_t* __restrict__ flag, int64_t N, int64_t E) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int32_t s = src[e], d = dst[e];
  if (s < 0 || s >= N || d < 0 || d >= N) {
    atomicOr(flag, 1);
    return;
  }
  atomicMax(flag + 1, atomicAdd(&counts[d], 1) + 1);
}

// Sort key of a CSR edge: (src, input index), unique per edge.
__device__ __forceinline__ uint64_t csr_key(int32_t s, int32_t e) {
  return (uint64_t(uint32_t(s)) << 32) | uint64_t(uint32_t(e));
}

__global__ void coo_scatter(const int32_t* __restrict__ src, const int32_t* __restrict__ dst,
                            const int32_t* __restrict__ row_ptr, int32_t* __restrict__ fill,
                            uint64_t* __restrict__ key, int32_t* __restrict__ seg, int64_t E) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const int32_t d = dst[e];
  const int32_t pos = row_ptr[d] + atomicAdd(&fill[d], 1);
  key[pos] = csr_key(src[e], int32_t(e));
  seg[pos] = d;
}

__global__ void csr_unpack(const uint64_t* __restrict__ key, int32_t* __restrict__ src_sorted,
                           int32_t* __restrict__ perm, int64_t E) {
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= E) return;
  const uint64_t v = key[k];
  src_sorted[k] = int32_t(v >> 32);
  perm[k] = int32_t(v & 0xffffffffu);
}

// ---- segmented sort of unique keys (positions never leave their segment)
constexpr int kRun = 256;

// Sort runs of kRun consecutive elements of each segment (the last run of a
// segment may be shorter): an element's place is the count of smaller keys.
__global__ void seg_sort_runs(const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg,
                              const uint64_t* __restrict__ in, uint64_t* __restrict__ out, int64_t n) {
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t d = seg[k];
  const int64_t lo = seg_ptr[d], hi = seg_ptr[d + 1];
  const int64_t r0 = lo + ((k - lo) / kRun) * kRun;
  const int64_t r1 = r0 + kRun < hi ? r0 + kRun : hi;
  const uint64_t v = in[k];
  int32_t rank = 0;
  for (int64_t j = r0; j < r1; ++j) rank += in[j] < v ? 1 : 0;
  out[r0 + rank] = v;
}

// Merge sorted runs of length R pairwise (runs 2i and 2i+1 of a segment).
__global__ void seg_merge_runs(const int32_t* __restrict__ seg_ptr, const int32_t* __restrict__ seg,
                               const uint64_t* __restrict__ in, uint64_t* __restrict__ out, int64_t n, int64_t R) {
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  const int32_t d = seg[k];
  const int64_t lo = seg_ptr[d], hi = seg_ptr[d + 1];
  const int64_t r = (k - lo) / R;
  const int64_t ps = lo + (r ^ 1) * R;
  const uint64_t v = in[k];
  if (ps >= hi) {  // no partner run: the element stays
    out[k] = v;
    return;
  }
  const int64_t pe = ps + R < hi ? ps + R : hi;
  int64_t a = ps, b = pe;  // first partner key not below v
  while (a < b) {
    const int64_t m = (a + b) >> 1;
    if (in[m] < v)
      a = m + 1;
    else
      b = m;
  }
  out[lo + (r & ~int64_t(1)) * R + (k - lo - r * R) + (a - ps)] = v;
}

// ---- validation and transpose
__global__ void validate_csr(const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ src,
                             int32_t* __restrict__ bad, int64_t N, int64_t E) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i <= N) {
    const int32_t r = row_ptr[i];
    if (i == 0 && r != 0) atomicOr(bad, 1);
    if (i == N && r != E) atomicOr(bad, 2);
    if (i < N && row_ptr[i + 1] < r) atomicOr(bad, 4);
    if (r < 0 || r > E) atomicOr(bad, 8);
  }
  if (i < E) {
    const int32_t s = src[i];
    if (s < 0 || s >= N) atomicOr(bad, 16);
  }
}

// Edges in [pe0, pe1) (the padding node's segment) are left out of the transpose.
__global__ void src_count(const int32_t* __restrict__ src, int32_t* __restrict__ counts, int64_t E, int64_t pe0,
                          int64_t pe1) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < E && (e < pe0 || e >= pe1)) atomicAdd(&counts[src[e]], 1);
}

// key of a transposed edge: its CSR position (unique)
__global__ void src_scatter(const int32_t* __restrict__ src, const int32_t* __restrict__ col_ptr,
                            int32_t* __restrict__ fill, int32_t* __restrict__ seg,
                            uint64_t* __restrict__ key, int64_t E, int64_t pe0, int64_t pe1) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= E || (e >= pe0 && e < pe1)) return;
  const int32_t s = src[e];
  const int32_t pos = col_ptr[s] + atomicAdd(&fill[s], 1);
  seg[pos] = s;
  key[pos] = uint64_t(e);
}

__global__ void key_to_i32(const uint64_t* __restrict__ key, int32_t* __restrict__ out, int64_t n) {
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k < n) out[k] = int32_t(key[k]);
}

__global__ void fill_dst(const int32_t* __restrict__ row_ptr, int32_t* __restrict__ dst, int64_t N) {
  const int64_t n = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (n >= N) return;
  for (int32_t e = row_ptr[n]; e < row_ptr[n + 1]; ++e) dst[e] = int32_t(n);
}

int32_t read_flag(const int32_t* dflag, hipStream_t s) {
  int32_t h = 0;
  CGTP_CHECK_HIP(hipMemcpyAsync(&h, dflag, sizeof(h), hipMemcpyDeviceToHost, s));
  CGTP_CHECK_HIP(hipStreamSynchronize(s));
  return h;
}

}  // namespace

void exclusive_scan_i32(const int32_t* counts, int32_t* out, int64_t n, hipStream_t s) {
  if (n > 0) {
    const int64_t tiles = (n + kScanTile - 1) / kScanTile;
    DevBuf tsum(size_t(tiles) * 4), toff(size_t(tiles + 1) * 4);
    hipLaunchKernelGGL(scan_tiles, dim3(unsigned(tiles)), dim3(kScanThreads), 0, s, counts, out,
                       tsum.as<int32_t>(), n);
    CGTP_CHECK_HIP(hipGetLastError());
    if (tiles > 1) {
      exclusive_scan_i32(tsum.as<int32_t>(), toff.as<int32_t>(), tiles, s);
      hipLaunchKernelGGL(scan_add, dim3(blocks_for(n, 256)), dim3(256), 0, s, out, toff.as<int32_t>(), n);
      CGTP_CHECK_HIP(hipGetLastError());
    }
    // the temporaries are freed on return: wait for the kernels that read them
    CGTP_CHECK_HIP(hipStreamSynchronize(s));
  }
  hipLaunchKernelGGL(scan_total, dim3(1), dim3(1), 0, s, out, counts, n);
  CGTP_CHECK_HIP(hipGetLastError());
}

namespace {

// Sort the unique keys of every segment of seg_ptr (key[k] lies in segment
// seg[k]); the result is in *a or *b, returned. max_deg bounds the segment
// lengths (it sets the number of merge passes).
uint64_t* segmented_sort(const int32_t* seg_ptr, const int32_t* seg, uint64_t* a, uint64_t* b, int64_t n,
                         int64_t max_deg, hipStream_t s) {
  if (n == 0) return a;
  hipLaunchKernelGGL(seg_sort_runs, dim3(blocks_for(n, 256)), dim3(256), 0, s, seg_ptr, seg, a, b, n);
  CGTP_CHECK_HIP(hipGetLastError());
  std::swap(a, b);
  for (int64_t R = kRun; R < max_deg; R *= 2) {
    hipLaunchKernelGGL(seg_merge_runs, dim3(blocks_for(n, 256)), dim3(256), 0, s, seg_ptr, seg, a, b, n, R);
    CGTP_CHECK_HIP(hipGetLastError());
    std::swap(a, b);
  }
  return a;
}

}  // namespace

void csr_from_coo_launch(int64_t N, int64_t E, const int32_t* src, const int32_t* dst,
                         int32_t* row_ptr, int32_t* src_sorted, int32_t* perm, hipStream_t s) {
  DevBuf counts(size_t(N + 1) * 4), flag(8);
  CGTP_CHECK_HIP(hipMemsetAsync(counts.p, 0, size_t(N + 1) * 4, s));
  CGTP_CHECK_HIP(hipMemsetAsync(flag.p, 0, 8, s));
  if (E > 0) {
    hipLaunchKernelGGL(coo_count, dim3(blocks_for(E, 256)), dim3(256), 0, s, src, dst,
                       counts.as<int32_t>(), flag.as<int32_t>(), N, E);
    CGTP_CHECK_HIP(hipGetLastError());
  }
  int32_t hflag[2] = {0, 0};
  CGTP_CHECK_HIP(hipMemcpyAsync(hflag, flag.p, sizeof(hflag), hipMemcpyDeviceToHost, s));
  CGTP_CHECK_HIP(hipStreamSynchronize(s));
  if (hflag[0]) throw Error{CGTP_ERR_INDEX, "csr_from_coo: src/dst outside [0, N)"};
  exclusive_scan_i32(counts.as<int32_t>(), row_ptr, N, s);
  if (E == 0) {
    CGTP_CHECK_HIP(hipStreamSynchronize(s));
    return;
  }
  DevBuf fill(size_t(N) * 4 + 4), seg(size_t(E) * 4), ka(size_t(E) * 8), kb(size_t(E) * 8);
  CGTP_CHECK_HIP(hipMemsetAsync(fill.p, 0, size_t(N) * 4 + 4, s));
  hipLaunchKernelGGL(coo_scatter, dim3(blocks_for(E, 256)), dim3(256), 0, s, src, dst, row_ptr,
                     fill.as<int32_t>(), ka.as<uint64_t>(), seg.as<int32_t>(), E);
  CGTP_CHECK_HIP(hipGetLastError());
  const uint64_t* sorted =
      segmented_sort(row_ptr, seg.as<int32_t>(), ka.as<uint64_t>(), kb.as<uint64_t>(), E, hflag[1], s);
  hipLaunchKernelGGL(csr_unpack, dim3(blocks_for(E, 256)), dim3(256), 0, s, sorted, src_sorted, perm, E);
  CGTP_CHECK_HIP(hipGetLastError());
  CGTP_CHECK_HIP(hipStreamSynchronize(s));
}

cgtp_graph_s* graph_create(int64_t N, int64_t E, const int32_t* row_ptr, const int32_t* src,
                           hipStream_t s, int32_t pad) {
  if (pad < -1 || (pad >= 0 && pad >= N)) throw Error{CGTP_ERR_INDEX, "graph_create: padding node outside [-1, N)"};
  auto g = std::make_unique<cgtp_graph_s>();
  g->N = N;
  g->E = E;
  g->row_ptr = row_ptr;
  g->src = src;
  g->pad = pad;
  CGTP_CHECK_HIP(hipGetDevice(&g->device));
  {
    DevBuf flag(4);
    CGTP_CHECK_HIP(hipMemsetAsync(flag.p, 0, 4, s));
    const int64_t n = (N + 1 > E ? N + 1 : E);
    hipLaunchKernelGGL(validate_csr, dim3(blocks_for(n, 256)), dim3(256), 0, s, row_ptr, src,
                       flag.as<int32_t>(), N, E);
    CGTP_CHECK_HIP(hipGetLastError());
    const int32_t bad = read_flag(flag.as<int32_t>(), s);
    if (bad)
      throw Error{CGTP_ERR_INDEX, "graph_create: invalid CSR (flags " + std::to_string(bad) +
                                      "): need row_ptr[0]=0, non-decreasing, row_ptr[N]=E, src in [0,N)"};
  }
  std::vector<int32_t> order;
  int64_t max_src_deg = 0;
  {
    std::vector<int32_t> hrp(static_cast<size_t>(N + 1));
    std::vector<int32_t> hsrc(static_cast<size_t>(E));
    CGTP_CHECK_HIP(hipMemcpyAsync(hrp.data(), row_ptr, size_t(N + 1) * 4, hipMemcpyDeviceToHost, s));
    if (E > 0) CGTP_CHECK_HIP(hipMemcpyAsync(hsrc.data(), src, size_t(E) * 4, hipMemcpyDeviceToHost, s));
    CGTP_CHECK_HIP(hipStreamSynchronize(s));
    order = receiver_schedule(N, hrp, hsrc);
    if (pad >= 0) {
      g->pad_e0 = hrp[size_t(pad)];
      g->pad_e1 = hrp[size_t(pad) + 1];
    }
    // largest source degree of the transpose (sets its merge passes)
    std::vector<int32_t> deg(size_t(N), 0);
    for (int64_t e = 0; e < E; ++e)
      if (e < g->pad_e0 || e >= g->pad_e1) max_src_deg = std::max<int64_t>(max_src_deg, ++deg[size_t(hsrc[size_t(e)])]);
  }
  CGTP_CHECK_HIP(hipMalloc(&g->col_ptr, size_t(N + 1) * 4));
  if (hipMalloc(&g->order, size_t(N) * 4 + 4) != hipSuccess) {
    (void)hipFree(g->col_ptr);
    throw Error{CGTP_ERR_ALLOC, "graph_create: device allocation failed"};
  }
  if (E > 0) {
    if (hipMalloc(&g->eid, size_t(E) * 4) != hipSuccess || hipMalloc(&g->dst, size_t(E) * 4) != hipSuccess) {
      (void)hipFree(g->col_ptr);
      (void)hipFree(g->order);
      (void)hipFree(g->eid);
      throw Error{CGTP_ERR_ALLOC, "graph_create: device allocation failed"};
    }
  }
  try {
    DevBuf counts(size_t(N + 1) * 4);
    CGTP_CHECK_HIP(hipMemsetAsync(counts.p, 0, size_t(N + 1) * 4, s));
    if (E > 0) {
      hipLaunchKernelGGL(src_count, dim3(blocks_for(E, 256)), dim3(256), 0, s, src, counts.as<int32_t>(), E,
                         g->pad_e0, g->pad_e1);
      CGTP_CHECK_HIP(hipGetLastError());
    }
    if (N > 0)
      CGTP_CHECK_HIP(hipMemcpyAsync(g->order, order.data(), size_t(N) * 4, hipMemcpyHostToDevice, s));
    exclusive_scan_i32(counts.as<int32_t>(), g->col_ptr, N, s);
    if (E > 0) {
      DevBuf fill(size_t(N) * 4 + 4), seg(size_t(E) * 4), ka(size_t(E) * 8), kb(size_t(E) * 8);
      CGTP_CHECK_HIP(hipMemsetAsync(fill.p, 0, size_t(N) * 4 + 4, s));
      hipLaunchKernelGGL(src_scatter, dim3(blocks_for(E, 256)), dim3(256), 0, s, src, g->col_ptr,
                         fill.as<int32_t>(), seg.as<int32_t>(), ka.as<uint64_t>(), E, g->pad_e0, g->pad_e1);
      CGTP_CHECK_HIP(hipGetLastError());
      const int64_t Et = g->E_t();
      if (Et > 0) {
        const uint64_t* sorted = segmented_sort(g->col_ptr, seg.as<int32_t>(), ka.as<uint64_t>(),
                                                kb.as<uint64_t>(), Et, max_src_deg, s);
        hipLaunchKernelGGL(key_to_i32, dim3(blocks_for(Et, 256)), dim3(256), 0, s, sorted, g->eid, Et);
        CGTP_CHECK_HIP(hipGetLastError());
      }
      hipLaunchKernelGGL(fill_dst, dim3(blocks_for(N, 256)), dim3(256), 0, s, row_ptr, g->dst, N);
      CGTP_CHECK_HIP(hipGetLastError());
    }
    CGTP_CHECK_HIP(hipStreamSynchronize(s));
  } catch (...) {
    (void)hipFree(g->col_ptr);
    (void)hipFree(g->order);
    (void)hipFree(g->eid);
    (void)hipFree(g->dst);
    throw;
  }
  return g.release();
}

void graph_destroy(cgtp_graph_s* g) {
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  if (hipSetDevice(g->device) == hipSuccess) {
    (void)hipFree(g->col_ptr);
    (void)hipFree(g->order);
    (void)hipFree(g->eid);
    (void)hipFree(g->dst);
  }
  if (have) (void)hipSetDevice(cur);
  delete g;
}

void graph_transpose_copy(const cgtp_graph_s* g, int32_t* col_ptr, int32_t* eid, hipStream_t s) {
  CGTP_CHECK_HIP(hipMemcpyAsync(col_ptr, g->col_ptr, size_t(g->N + 1) * 4, hipMemcpyDeviceToDevice, s));
  if (g->E_t() > 0)
    CGTP_CHECK_HIP(hipMemcpyAsync(eid, g->eid, size_t(g->E_t()) * 4, hipMemcpyDeviceToDevice, s));
}

}  // namespace cgtp
