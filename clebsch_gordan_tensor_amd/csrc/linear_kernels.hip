// Equivariant linear map (channel mixing) on the matrix cores.
//
// What is computed: linear mixing of channels within each irrep type, one of
// the core operations listed in "E3J: An Efficient and Open-Source Backend for
// Euclidean Equivariant Operations on GPU and TPU", appendix A.3 (the weights
// of such learnable layers: MolSSI e3nn course, lesson 03b):
//   out[z, o, m, v] = sum over paths p = (i, o) of sum_u x[z, i, m, u] W_p[u, v]
// for every (input block i, output block o) with the same l and parity, W_p
// stored [u][v] row-major, paths input-major. For one path and one m this is
// the product of a [rows x u] matrix (row stride dim_in) with W_p: a dense
// contraction, so it runs on v_mfma_f32_16x16x4_f32 (fp32 products and sums;
// bf16 storage is widened exactly to fp32 on load).
//
// Forward and grad_x share one kernel over "jobs": a job is a run of at most
// 128 output columns of one block and one m, fed by one or more terms (an A
// block of the row times a weight matrix read with given strides). A
// workgroup takes 128 rows of one job; a wave 32 rows x 128 columns (16 MFMA
// tiles). grad_W = x^T g summed over rows and m: a workgroup takes one row
// chunk of one (path, 128 x 128 weight tile), a wave 32 weight rows x 128
// columns; per-chunk partials are added over the chunks in a fixed order by a
// second kernel (no atomics, bitwise reproducible).
//
// MFMA lane layout (checked on the device): lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16] and holds D[4 (l / 16) + r][l % 16], r = 0..3. Within
// a 16-wide slice of the contraction, lane slot k = l / 16 of step j takes
// contraction index 4k + j, so each lane reads 4 consecutive A values at once.
#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <type_traits>
#include <vector>

#include "device_util.hpp"
#include "linear.hpp"

namespace cgtp {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

struct LinTerm {  // C[row, n] += sum_k A[row, a_off + k] * W[b_off + k * b_sk + (b_n0 + n) * b_sn]
  int32_t a_off, K, b_off, b_sk, b_sn, pad0, pad1, pad2;
};
struct LinJob {  // output columns c_off .. c_off + n_len of every row; terms t0 .. t1
  int32_t c_off, n_len, b_n0, t0, t1, pad0, pad1, pad2;
};
struct LinDW {  // weight tile [u0, u0 + 128) x [v0, v0 + 128) of one path
  int32_t x_off, mu, g_off, mv, nm, w_off, u0, v0;
};

#ifndef CGTP_LINEAR_BF16_MFMA
#define CGTP_LINEAR_BF16_MFMA 1
#endif

constexpr int kLinThreads = 256;
constexpr int kLinRows = 128;  // rows per workgroup of the row kernel (4 waves x 32)
constexpr int kLinCols = 128;  // columns per job
constexpr int kLinURows = 128;  // weight rows per workgroup of the grad_W kernel

template <typename T>
__device__ __forceinline__ float ld1(const T* p) {
  return to_acc<float>(*p);
}

// Guarded load as an unconditional load of an in-bounds element (the caller
// clamps the index) followed by a select: a load under a branch would be
// waited for before the next one is issued.
template <typename T>
__device__ __forceinline__ float ld_sel(const T* p, bool ok) {
  const float v = ld1(p);
  return ok ? v : 0.f;
}

// Four consecutive elements of one row, as stored; widened to fp32 at use.
template <typename T>
struct Quad;
template <>
struct Quad<float> {
  typedef float V __attribute__((ext_vector_type(4)));
  V v;
  __device__ static __forceinline__ Quad load4(const float* p) { return Quad{*reinterpret_cast<const V*>(p)}; }
  __device__ __forceinline__ void set(int j, const float* p) { v[j] = *p; }
  __device__ __forceinline__ float get(int j) const { return v[j]; }
};
template <>
struct Quad<bf16> {
  typedef uint16_t V __attribute__((ext_vector_type(4)));
  V v;
  __device__ static __forceinline__ Quad load4(const bf16* p) { return Quad{*reinterpret_cast<const V*>(p)}; }
  __device__ __forceinline__ void set(int j, const bf16* p) { v[j] = p->bits; }
  __device__ __forceinline__ float get(int j) const { return bf16_to_f32(v[j]); }
};

// B (the weight matrix of a term) goes through LDS in chunks of 16
// contraction rows x 128 columns, double-buffered: the next chunk's global
// loads are in flight while the MFMAs run on the current one.
constexpr int kKC = 16;          // contraction rows per B chunk
constexpr int kBP = kLinCols + 4;  // padded LDS row (lanes of 4 k-slots land in different banks)

template <typename T, bool AVEC>
__global__ __launch_bounds__(kLinThreads) void lin_rows_kernel(const T* __restrict__ A, int64_t lda,
                                                             const T* __restrict__ W, T* __restrict__ C,
                                                             int64_t ldcr, int64_t rows,
                                                             const LinJob* __restrict__ jobs,
                                                             const LinTerm* __restrict__ terms, int njobs) {
  __shared__ float bs[2][kKC * kBP];
  const LinJob jb = ldc(jobs + blockIdx.x % unsigned(njobs));
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int64_t r0 = int64_t(blockIdx.x / unsigned(njobs)) * kLinRows + wave * 32;  // two 16-row tiles per wave
  int64_t arow[2];
  bool row_ok[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    arow[s] = r0 + 16 * s + li;
    row_ok[s] = arow[s] < rows;
  }
  v4f acc[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  constexpr int PER = kKC * kLinCols / kLinThreads;  // staged values per thread and chunk
  for (int t = jb.t0; t < jb.t1; ++t) {
    const LinTerm tm = ldc(terms + t);
    const T* __restrict__ wb = W + tm.b_off + int64_t(jb.b_n0) * tm.b_sn;
    const bool kfast = tm.b_sk == 1;  // transposed weights: walk k fastest for contiguous reads
    const int nch = (tm.K + kKC - 1) / kKC;
    // B chunk staging: fetch() requests the elements as stored (clamped
    // in-bounds indexes, nothing depends on the loads yet), stash() widens,
    // masks and writes them to LDS.
    T pre[PER];
    auto fetch = [&](int c) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int e = int(threadIdx.x) + q * kLinThreads;
        const int kk = kfast ? (e % kKC) : (e / kLinCols), n = kfast ? (e / kKC) : (e % kLinCols);
        const int k = c * kKC + kk;
        pre[q] = wb[int64_t(k < tm.K ? k : 0) * tm.b_sk + int64_t(n < jb.n_len ? n : 0) * tm.b_sn];
      }
    };
    auto stash = [&](int c, int buf) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        const int e = int(threadIdx.x) + q * kLinThreads;
        const int kk = kfast ? (e % kKC) : (e / kLinCols), n = kfast ? (e / kKC) : (e % kLinCols);
        const bool ok = c * kKC + kk < tm.K && n < jb.n_len;
        bs[buf][kk * kBP + n] = ok ? ld1(&pre[q]) : 0.f;
      }
    };
    // This lane's A elements of one chunk, [k16 half][row tile] x 4 consecutive
    // k, kept as loaded (no dependent instruction, so the loads stay in flight
    // during the previous chunk's MFMAs) and widened and masked at use. Rows
    // past the end read row 0 (their results are not stored: row i of an MFMA
    // product depends on row i of A only); k past K reads element 0 and is
    // masked to zero at use.
    auto load_a = [&](int c, Quad<T> (&a)[kKC / 16][2]) {
#pragma unroll
      for (int h = 0; h < kKC / 16; ++h) {
        const int ka = c * kKC + 16 * h + 4 * lk;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const T* __restrict__ ar = A + (row_ok[s2] ? arow[s2] : int64_t(0)) * lda + tm.a_off;
          if (AVEC) {
            a[h][s2] = Quad<T>::load4(ar + (ka < tm.K ? ka : 0));
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) a[h][s2].set(j, ar + (ka + j < tm.K ? ka + j : 0));
          }
        }
      }
    };
    __syncthreads();  // the previous term's last chunk is consumed
    // Per chunk: the next chunk's operands are requested first, without a
    // condition (past the last chunk the clamped requests read in-bounds
    // elements that are masked to zero and never used; a conditional request
    // could be moved behind the MFMAs by the compiler), the MFMAs run on the
    // current chunk, then the next B chunk goes to the other LDS buffer.
    Quad<T> ac[kKC / 16][2], an[kKC / 16][2];
    fetch(0);
    load_a(0, ac);
    stash(0, 0);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      fetch(c + 1);
      load_a(c + 1, an);
      __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
      const float* __restrict__ bc = bs[c & 1];
#pragma unroll
      for (int h = 0; h < kKC / 16; ++h) {
        const int ka = c * kKC + 16 * h + 4 * lk;
        float av[2][4];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int j = 0; j < 4; ++j) av[s2][j] = ka + j < tm.K ? ac[h][s2].get(j) : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float* __restrict__ br = bc + (16 * h + 4 * lk + j) * kBP + li;
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const float b = br[tt * 16];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
              acc[s2][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[s2][j], b, acc[s2][tt], 0, 0, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // the requests complete behind the MFMAs
      stash(c + 1, (c + 1) & 1);
#pragma unroll
      for (int h = 0; h < kKC / 16; ++h)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) ac[h][s2] = an[h][s2];
      __syncthreads();
    }
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int n = tt * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + 16 * s + 4 * lk + r;
        if (row < rows && n < jb.n_len) from_acc(C[row * ldcr + jb.c_off + n], acc[s][tt][r]);
      }
    }
}

// bf16 storage with every offset, width and row stride a multiple of 8: the
// products run on v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in
// fp32 and accumulate in fp32, so the result matches widening to fp32 first
// up to summation order). Lane l supplies A[l % 16][8 (l / 16) + j] and
// B[8 (l / 16) + j][l % 16], j < 8 (checked on the device), so each lane
// loads 8 consecutive k of its row in one 16-byte load, and the B chunk sits
// in LDS n-major ([n][k]) so each lane reads its 8 k values in one access.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
constexpr int kKB = 32;         // contraction rows per B chunk (the MFMA's K)
constexpr int kBTP = kKB + 8;   // padded n-major LDS row of a B chunk, in elements
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// n-major LDS tiles T[n][k] (rows of kBTP elements: 32 k and 16 bytes of
// padding) hold their 16-byte k runs (k = 8c .. 8c + 7) at run position
// c ^ ((n >> 3) & 3). With the 80-byte rows, any 8 consecutive n read at one
// run position, and the transposing writes below (8 lanes with consecutive
// column blocks and one row block), land in 8 different groups of 4 banks.
__device__ __forceinline__ int tile_run(int n, int c) { return n * kBTP + 8 * (c ^ ((n >> 3) & 3)); }

// Transposing stash of one block of a row-major (k slow) bf16 tile: R[r]
// holds W consecutive n of row k = 8 kb + r (W = 2 or 4, packed two per
// dword); each of the W columns n0 + j goes to T[n0 + j][8 kb .. 8 kb + 7]
// as one 16-byte write.
template <int W>
__device__ __forceinline__ void stash_block(uint16_t* __restrict__ T, int n0, int kb, const uint32_t (&R)[8][W / 2]) {
#pragma unroll
  for (int j = 0; j < W; ++j) {
    const int d = j >> 1;
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = R[2 * p][d], hi = R[2 * p + 1][d];
      o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    *reinterpret_cast<u32x4*>(T + tile_run(n0 + j, kb)) = o;
  }
}

// One workgroup = 128 rows (4 waves x 32) x the 128 output columns of one job.
// The contraction runs in super-chunks of kSC B chunks (128 k): every global
// load of a super-chunk (the lane's A runs and its share of the B chunks) is
// issued before any is used, so with K <= 128 a workgroup waits for one
// memory round trip, not one per chunk (the kernel is latency-bound: few
// MFMAs per byte).
constexpr int kSC = 4;  // B chunks per super-chunk

__global__ __launch_bounds__(kLinThreads) __attribute__((amdgpu_waves_per_eu(3))) void lin_rows_bf16_kernel(const bf16* __restrict__ A, int64_t lda,
                                                                  const bf16* __restrict__ W, bf16* __restrict__ C,
                                                                  int64_t ldcr, int64_t rows,
                                                                  const LinJob* __restrict__ jobs,
                                                                  const LinTerm* __restrict__ terms, int njobs,
                                                                  int cvec) {
  __shared__ __attribute__((aligned(16))) uint16_t bt[kSC][kLinCols * kBTP];
  const LinJob jb = ldc(jobs + blockIdx.x % unsigned(njobs));
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int64_t r0 = int64_t(blockIdx.x / unsigned(njobs)) * kLinRows + wave * 32;  // two 16-row tiles per wave
  // this lane's two A rows (rows past the end read row 0; their results are
  // not stored)
  const uint16_t* arp[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int64_t ar = r0 + 16 * s + li;
    arp[s] = reinterpret_cast<const uint16_t*>(A) + (ar < rows ? ar : int64_t(0)) * lda;
  }
  v4f acc[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  const u16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  const int bn = 2 * (int(threadIdx.x) & 63), bk = int(threadIdx.x) >> 6;  // runs along n: block origin
  for (int t = jb.t0; t < jb.t1; ++t) {
    const LinTerm tm = ldc(terms + t);
    const uint16_t* __restrict__ wb =
        reinterpret_cast<const uint16_t*>(W) + tm.b_off + int64_t(jb.b_n0) * tm.b_sn;
    const bool kfast = tm.b_sk == 1;  // transposed weights: runs of 8 along k
    for (int kb = 0; kb < tm.K; kb += kSC * kKB) {
      // Requests, unconditional from clamped addresses (masked when used or
      // stashed). A: 8 consecutive k of each of the lane's two rows per chunk
      // (K is a multiple of 8, so a run is wholly inside or past K). B chunk,
      // 32 x 128: with runs along k (transposed weights), 512 runs of 8, two
      // per thread, stored as they are; with runs along n, one 8 (k) x 2 (n)
      // block per thread, transposed on the way into LDS.
      u16x8 a[kSC][2];
      uint32_t wv[kSC][8];  // the thread's B values of each chunk, as loaded (either layout)
#pragma unroll
      for (int c = 0; c < kSC; ++c) {
        const int ka = kb + c * kKB + 8 * lk;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          a[c][s2] = *reinterpret_cast<const u16x8*>(arp[s2] + tm.a_off + (ka < tm.K ? ka : 0));
        if (kfast) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int u = int(threadIdx.x) + q * kLinThreads, n = u >> 2, k = kb + c * kKB + (u & 3) * 8;
            const bool ok = k < tm.K && n < jb.n_len;
            const u32x4 v = *reinterpret_cast<const u32x4*>(wb + (ok ? k : 0) + int64_t(ok ? n : 0) * tm.b_sn);
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[c][4 * q + j] = v[j];
          }
        } else {
          const int k0 = kb + c * kKB + 8 * bk;
          const bool ok = k0 < tm.K && bn < jb.n_len;
          const uint16_t* __restrict__ bp = wb + int64_t(ok ? k0 : 0) * tm.b_sk + (ok ? bn : 0);
#pragma unroll
          for (int r = 0; r < 8; ++r) wv[c][r] = *reinterpret_cast<const uint32_t*>(bp + int64_t(r) * tm.b_sk);
        }
      }
      __syncthreads();  // the previous super-chunk's B tiles are consumed
#pragma unroll
      for (int c = 0; c < kSC; ++c) {
        if (kfast) {
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int u = int(threadIdx.x) + q * kLinThreads, n = u >> 2, k = kb + c * kKB + (u & 3) * 8;
            const bool ok = k < tm.K && n < jb.n_len;
            u32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = ok ? wv[c][4 * q + j] : 0u;
            *reinterpret_cast<u32x4*>(&bt[c][tile_run(n, u & 3)]) = v;
          }
        } else {
          uint32_t m[8][1];
          const bool ok = kb + c * kKB + 8 * bk < tm.K && bn < jb.n_len;
#pragma unroll
          for (int r = 0; r < 8; ++r) m[r][0] = ok ? wv[c][r] : 0u;
          stash_block<2>(bt[c], bn, bk, m);
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < kSC; ++c) {
        if (kb + c * kKB >= tm.K) break;  // uniform: chunks past K
        const bool kin = kb + c * kKB + 8 * lk < tm.K;
        bf16x8 av[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) av[s2] = __builtin_bit_cast(bf16x8, kin ? a[c][s2] : zero8);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const bf16x8 bv =
              __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(&bt[c][tile_run(tt * 16 + li, lk)]));
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            acc[s2][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s2], bv, acc[s2][tt], 0, 0, 0);
        }
      }
    }
  }
  if (cvec) {
    // 16-row halves of the wave's tile through LDS, so each lane stores 8
    // consecutive columns of a row with one 16-byte write
    constexpr int kCP = kLinCols + 8;  // padded row of the staged tile, in elements
    static_assert((kLinThreads / 64) * 16 * kCP <= kSC * kLinCols * kBTP, "staged tiles fit the B buffers");
    uint16_t* __restrict__ tile = &bt[0][0] + wave * (16 * kCP);
    __syncthreads();  // every wave's MFMAs have read their last B tile
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile[(4 * lk + r) * kCP + tt * 16 + li] = f32_to_bf16(acc[s][tt][r]);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = lane + 64 * i, row = q >> 4, n = (q & 15) * 8;
        const int64_t grow = r0 + 16 * s + row;
        const u16x8 v = *reinterpret_cast<const u16x8*>(tile + row * kCP + n);
        if (grow < rows && n < jb.n_len)
          *reinterpret_cast<u16x8*>(reinterpret_cast<uint16_t*>(C) + grow * ldcr + jb.c_off + n) = v;
      }
      __syncthreads();
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int n = tt * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = r0 + 16 * s + 4 * lk + r;
        if (row < rows && n < jb.n_len) from_acc(C[row * ldcr + jb.c_off + n], acc[s][tt][r]);
      }
    }
}

template <typename T>
__global__ __launch_bounds__(kLinThreads) void lin_dw_kernel(const T* __restrict__ X, int64_t ldx,
                                                           const T* __restrict__ G, int64_t ldg,
                                                           float* __restrict__ part, int64_t w_numel,
                                                           int64_t rows, int64_t rows_per_chunk,
                                                           const LinDW* __restrict__ jobs) {
  const LinDW jb = ldc(jobs + blockIdx.y);
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int64_t z0 = int64_t(blockIdx.x) * rows_per_chunk;
  const int64_t z1 = z0 + rows_per_chunk < rows ? z0 + rows_per_chunk : rows;
  const int ub = jb.u0 + 32 * wave;
  v4f acc[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  if (ub < jb.mu) {
    constexpr int QU = 4;  // row quads whose operands are loaded before their MFMAs run
    for (int m = 0; m < jb.nm; ++m) {
      for (int64_t zq = z0; zq < z1; zq += 4 * QU) {
        float a[QU][2], b[QU][8];
#pragma unroll
        for (int q = 0; q < QU; ++q) {
          const int64_t zr = zq + 4 * q + lk;  // this lane's contraction slot is a row
          const bool ok = zr < z1;
          const T* __restrict__ xr = X + (ok ? zr : z0) * ldx + jb.x_off + int64_t(m) * jb.mu;
          const T* __restrict__ gr = G + (ok ? zr : z0) * ldg + jb.g_off + int64_t(m) * jb.mv;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const int u = ub + 16 * s + li;
            a[q][s] = ld_sel(xr + (u < jb.mu ? u : 0), ok && u < jb.mu);
          }
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const int v = jb.v0 + 16 * tt + li;
            b[q][tt] = ld_sel(gr + (v < jb.mv ? v : 0), ok && v < jb.mv);
          }
        }
#pragma unroll
        for (int q = 0; q < QU; ++q)
#pragma unroll
          for (int tt = 0; tt < 8; ++tt)
#pragma unroll
            for (int s = 0; s < 2; ++s)
              acc[s][tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q][s], b[q][tt], acc[s][tt], 0, 0, 0);
      }
    }
  }
  float* __restrict__ pc = part + int64_t(blockIdx.x) * w_numel + jb.w_off;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = ub + 16 * s + 4 * lk + r, v = jb.v0 + 16 * tt + li;
        if (u < jb.mu && v < jb.mv) pc[int64_t(u) * jb.mv + v] = acc[s][tt][r];
      }
}

// grad_W partials with bf16 storage on v_mfma_f32_16x16x32_bf16: the
// contraction runs over rows, which are strided in memory, so each 32-row
// step stages x and g transposed in LDS ([u][row] and [v][row]: each thread
// loads an 8-row x 4-column block with 8-byte row loads and writes its four
// columns as 16-byte runs, at the swizzled positions of tile_run) and every
// lane then reads its 8 consecutive rows of one u (A) and one v (B) in one
// access. Widths and offsets are multiples of 8.
__global__ __launch_bounds__(kLinThreads) void lin_dw_bf16_kernel(const bf16* __restrict__ X, int64_t ldx,
                                                                const bf16* __restrict__ G, int64_t ldg,
                                                                float* __restrict__ part, int64_t w_numel,
                                                                int64_t rows, int64_t rows_per_chunk,
                                                                const LinDW* __restrict__ jobs) {
  __shared__ __attribute__((aligned(16))) uint16_t xt[2][kLinURows * kBTP];
  __shared__ __attribute__((aligned(16))) uint16_t gt[2][kLinCols * kBTP];
  const LinDW jb = ldc(jobs + blockIdx.y);
  const int lane = int(threadIdx.x & 63), wave = int(threadIdx.x >> 6);
  const int li = lane & 15, lk = lane >> 4;
  const int64_t z0 = int64_t(blockIdx.x) * rows_per_chunk;
  const int64_t z1 = z0 + rows_per_chunk < rows ? z0 + rows_per_chunk : rows;
  const int ub = 32 * wave;  // this wave's weight rows within the tile
  v4f acc[2][8];
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[s][t] = v4f{0.f, 0.f, 0.f, 0.f};
  const uint16_t* __restrict__ Xs = reinterpret_cast<const uint16_t*>(X);
  const uint16_t* __restrict__ Gs = reinterpret_cast<const uint16_t*>(G);
  // one 32-row step: threads 0-127 take one 8 (row) x 4 (u) block of x each,
  // threads 128-255 one 8 x 4 block of g, requested from clamped addresses,
  // masked and transposed when stashed
  const bool tg = threadIdx.x >= 128;
  const int bc = 4 * (int(threadIdx.x) & 31), bz = (int(threadIdx.x) >> 5) & 3;  // block origin (column, row block)
  const int mlim = tg ? jb.mv : jb.mu, c0 = tg ? jb.v0 : jb.u0;
  const bool col_ok = c0 + bc < mlim;
  uint32_t pr[8][2];
  const int nsteps = int((z1 - z0 + kKB - 1) / kKB);
  const int total = jb.nm * nsteps;
  auto fetch = [&](int it) {
    const int m = it < total ? it / nsteps : 0;
    const int64_t zs = z0 + int64_t(it - m * nsteps) * kKB;
    const uint16_t* __restrict__ base = tg ? Gs + jb.g_off + int64_t(m) * jb.mv : Xs + jb.x_off + int64_t(m) * jb.mu;
    const int64_t ld = tg ? ldg : ldx;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t z = zs + 8 * bz + r;
      const bool ok = it < total && z < z1;
      const uint2 v = *reinterpret_cast<const uint2*>(base + (ok ? z : z0) * ld + (col_ok ? c0 + bc : 0));
      pr[r][0] = v.x;
      pr[r][1] = v.y;
    }
  };
  auto stash = [&](int it, int buf) {
    const int m = it < total ? it / nsteps : 0;
    const int64_t zs = z0 + int64_t(it - m * nsteps) * kKB;
    uint32_t q[8][2];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const bool ok = it < total && zs + 8 * bz + r < z1 && col_ok;
      q[r][0] = ok ? pr[r][0] : 0u;
      q[r][1] = ok ? pr[r][1] : 0u;
    }
    stash_block<4>(tg ? gt[buf] : xt[buf], bc, bz, q);
  };
  if (total > 0) {
    fetch(0);
    stash(0, 0);
    __syncthreads();
    for (int it = 0; it < total; ++it) {
      fetch(it + 1);
      __builtin_amdgcn_sched_barrier(0);  // keep the requests ahead of the MFMAs
      const uint16_t* __restrict__ xc = xt[it & 1];
      const uint16_t* __restrict__ gc = gt[it & 1];
      bf16x8 av[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        av[s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(xc + tile_run(ub + 16 * s2 + li, lk)));
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(gc + tile_run(16 * tt + li, lk)));
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          acc[s2][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[s2], bv, acc[s2][tt], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // the requests complete behind the MFMAs
      stash(it + 1, (it + 1) & 1);
      __syncthreads();
    }
  }
  float* __restrict__ pc = part + int64_t(blockIdx.x) * w_numel + jb.w_off;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int u = jb.u0 + ub + 16 * s + 4 * lk + r, v = jb.v0 + 16 * tt + li;
        if (u < jb.mu && v < jb.mv) pc[int64_t(u) * jb.mv + v] = acc[s][tt][r];
      }
}

// grad_W[j] = sum over chunks c (ascending) of part[c][j]
template <typename T>
__global__ __launch_bounds__(kLinThreads) void lin_colsum_kernel(const float* __restrict__ part, T* __restrict__ out,
                                                               int64_t nchunks, int64_t w_numel) {
  const int64_t j = int64_t(blockIdx.x) * kLinThreads + threadIdx.x;
  if (j >= w_numel) return;
  float s = 0.f;
  for (int64_t c = 0; c < nchunks; ++c) s += part[c * w_numel + j];
  from_acc(out[j], s);
}

struct LinTables {
  LinJob* fjobs = nullptr;
  LinTerm* fterms = nullptr;
  LinJob* xjobs = nullptr;
  LinTerm* xterms = nullptr;
  LinDW* wjobs = nullptr;
  int nf = 0, nx = 0, nw = 0;
  bool avec_f = true, avec_x = true;  // 4-aligned A offsets and K (row strides checked per call)
  bool v8_f = true, v8_x = true, v8_w = true;  // offsets and widths multiples of 8 (bf16 matrix-core kernels)
  bool c8_f = true, c8_x = true;  // output column runs of the row jobs start and end at multiples of 8
};

std::mutex g_lin_mu;
std::map<std::pair<const cgtp_linear_s*, int>, LinTables> g_lin_tables;

template <typename X>
X* upload(const std::vector<X>& v) {
  X* p = nullptr;
  CGTP_CHECK_HIP(hipMalloc(&p, std::max<size_t>(v.size(), 1) * sizeof(X)));
  if (!v.empty()) CGTP_CHECK_HIP(hipMemcpy(p, v.data(), v.size() * sizeof(X), hipMemcpyHostToDevice));
  return p;
}

const LinTables& lin_tables(const cgtp_linear_s* lin) {
  int dev = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lock(g_lin_mu);
  auto it = g_lin_tables.find({lin, dev});
  if (it != g_lin_tables.end()) return it->second;
  LinTables t;
  std::vector<LinJob> fj, xj;
  std::vector<LinTerm> ft, xt;
  std::vector<LinDW> wj;
  // forward: output block o, component m, column run n0
  for (size_t o = 0; o < lin->O.size(); ++o) {
    const int mv = lin->O[o].mul, nm = 2 * lin->O[o].l + 1;
    for (int m = 0; m < nm; ++m)
      for (int n0 = 0; n0 < mv; n0 += kLinCols) {
        LinJob j{int32_t(lin->out_off[o] + int64_t(m) * mv + n0), std::min(kLinCols, mv - n0), n0,
                 int32_t(ft.size()), 0, 0, 0, 0};
        for (const auto& p : lin->paths)
          if (p.o == int(o)) {
            const int64_t a_off = lin->in_off[size_t(p.i)] + int64_t(m) * p.mu;
            ft.push_back(LinTerm{int32_t(a_off), p.mu, int32_t(p.w_off), p.mv, 1, 0, 0, 0});
            t.avec_f = t.avec_f && a_off % 4 == 0 && p.mu % 4 == 0;
            t.v8_f = t.v8_f && a_off % 8 == 0 && p.mu % 8 == 0 && p.mv % 8 == 0 && p.w_off % 8 == 0;
          }
        j.t1 = int32_t(ft.size());
        t.c8_f = t.c8_f && j.c_off % 8 == 0 && j.n_len % 8 == 0;
        fj.push_back(j);
      }
  }
  // grad_x: input block i, component m, column run n0; B[k = v][n = u] = W_p[u][v]
  for (size_t i = 0; i < lin->I.size(); ++i) {
    const int mu = lin->I[i].mul, nm = 2 * lin->I[i].l + 1;
    for (int m = 0; m < nm; ++m)
      for (int n0 = 0; n0 < mu; n0 += kLinCols) {
        LinJob j{int32_t(lin->in_off[i] + int64_t(m) * mu + n0), std::min(kLinCols, mu - n0), n0,
                 int32_t(xt.size()), 0, 0, 0, 0};
        for (const auto& p : lin->paths)
          if (p.i == int(i)) {
            const int64_t a_off = lin->out_off[size_t(p.o)] + int64_t(m) * p.mv;
            xt.push_back(LinTerm{int32_t(a_off), p.mv, int32_t(p.w_off), 1, p.mv, 0, 0, 0});
            t.avec_x = t.avec_x && a_off % 4 == 0 && p.mv % 4 == 0;
            t.v8_x = t.v8_x && a_off % 8 == 0 && p.mu % 8 == 0 && p.mv % 8 == 0 && p.w_off % 8 == 0;
          }
        j.t1 = int32_t(xt.size());
        t.c8_x = t.c8_x && j.c_off % 8 == 0 && j.n_len % 8 == 0;
        xj.push_back(j);
      }
  }
  // grad_W: path, weight tile
  for (const auto& p : lin->paths)
    for (int u0 = 0; u0 < p.mu; u0 += kLinURows)
      for (int v0 = 0; v0 < p.mv; v0 += kLinCols)
        wj.push_back(LinDW{int32_t(lin->in_off[size_t(p.i)]), p.mu, int32_t(lin->out_off[size_t(p.o)]), p.mv,
                           2 * p.l + 1, int32_t(p.w_off), u0, v0});
  for (const auto& p : lin->paths)
    t.v8_w = t.v8_w && p.mu % 8 == 0 && p.mv % 8 == 0 && lin->in_off[size_t(p.i)] % 8 == 0 &&
             lin->out_off[size_t(p.o)] % 8 == 0;
  t.fjobs = upload(fj);
  t.fterms = upload(ft);
  t.xjobs = upload(xj);
  t.xterms = upload(xt);
  t.wjobs = upload(wj);
  t.nf = int(fj.size());
  t.nx = int(xj.size());
  t.nw = int(wj.size());
  return g_lin_tables.emplace(std::make_pair(lin, dev), t).first->second;
}

bool aligned16(const void* p, size_t bytes) { return reinterpret_cast<uintptr_t>(p) % bytes == 0; }

int64_t dw_rows_per_chunk(int64_t B) {
  int64_t r = std::max<int64_t>(1024, (B + 511) / 512);
  return (r + 3) / 4 * 4;
}
int64_t dw_chunks(int64_t B) { return B == 0 ? 0 : (B + dw_rows_per_chunk(B) - 1) / dw_rows_per_chunk(B); }

// Workgroups of the row kernels take (row tile, job) with the job fastest: the
// jobs of one row tile run side by side, so each tile's rows are read and
// written whole (every job covers one slice of a row) while their DRAM pages
// are open, rather than one slice per row across the whole matrix at a time.
dim3 rows_grid(int64_t rows, int njobs) {
  const int64_t n = (rows + kLinRows - 1) / kLinRows * int64_t(njobs);
  if (n > int64_t(UINT32_MAX)) throw Error{CGTP_ERR_UNSUPPORTED, "linear map: too many rows for one launch"};
  return dim3(unsigned(n));
}

template <typename T>
void rows_launch(const T* A, int64_t lda, const T* W, T* C, int64_t ldc, int64_t rows, const LinJob* jobs,
                 const LinTerm* terms, int njobs, bool avec, hipStream_t s) {
  if (rows == 0 || njobs == 0) return;
  const dim3 grid = rows_grid(rows, njobs);
  if (avec)
    hipLaunchKernelGGL((lin_rows_kernel<T, true>), grid, dim3(kLinThreads), 0, s, A, lda, W, C, ldc, rows, jobs,
                       terms, njobs);
  else
    hipLaunchKernelGGL((lin_rows_kernel<T, false>), grid, dim3(kLinThreads), 0, s, A, lda, W, C, ldc, rows, jobs,
                       terms, njobs);
  CGTP_CHECK_HIP(hipGetLastError());
}

// bf16 with 8-aligned offsets, widths and row strides: the bf16 matrix-core kernel
// (16-byte output stores when every job's column run and the output rows are
// 8-aligned)
bool rows_bf16_mfma(const void* A, int64_t lda, const void* W, void* C, int64_t ldcr, int64_t rows,
                    const LinJob* jobs, const LinTerm* terms, int njobs, bool v8, bool c8, hipStream_t s) {
  if (!v8 || lda % 8 != 0 || !aligned16(A, 16) || !aligned16(W, 16) || CGTP_LINEAR_BF16_MFMA == 0) return false;
  if (rows == 0 || njobs == 0) return true;
  const dim3 grid = rows_grid(rows, njobs);
  const int cvec = c8 && ldcr % 8 == 0 && aligned16(C, 16) ? 1 : 0;
  hipLaunchKernelGGL(lin_rows_bf16_kernel, grid, dim3(kLinThreads), 0, s, static_cast<const bf16*>(A), lda,
                     static_cast<const bf16*>(W), static_cast<bf16*>(C), ldcr, rows, jobs, terms, njobs, cvec);
  CGTP_CHECK_HIP(hipGetLastError());
  return true;
}

template <typename T>
void forward_typed(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, void* out, hipStream_t s) {
  const LinTables& t = lin_tables(lin);
  if (std::is_same<T, bf16>::value &&
      rows_bf16_mfma(x, lin->dim_in, w, out, lin->dim_out, B, t.fjobs, t.fterms, t.nf, t.v8_f, t.c8_f, s))
    return;
  const bool avec = t.avec_f && lin->dim_in % 4 == 0 && aligned16(x, 4 * sizeof(T));
  rows_launch<T>(static_cast<const T*>(x), lin->dim_in, static_cast<const T*>(w), static_cast<T*>(out), lin->dim_out,
                 B, t.fjobs, t.fterms, t.nf, avec, s);
}

template <typename T>
void backward_typed(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, const void* g, void* dx,
                    void* dw, void* ws, hipStream_t s) {
  const LinTables& t = lin_tables(lin);
  if (dx && std::is_same<T, bf16>::value &&
      rows_bf16_mfma(g, lin->dim_out, w, dx, lin->dim_in, B, t.xjobs, t.xterms, t.nx, t.v8_x, t.c8_x, s))
    dx = nullptr;  // done
  if (dx) {
    const bool avec = t.avec_x && lin->dim_out % 4 == 0 && aligned16(g, 4 * sizeof(T));
    rows_launch<T>(static_cast<const T*>(g), lin->dim_out, static_cast<const T*>(w), static_cast<T*>(dx),
                   lin->dim_in, B, t.xjobs, t.xterms, t.nx, avec, s);
  }
  if (dw && lin->w_numel > 0) {
    const int64_t nch = dw_chunks(B);
    float* part = static_cast<float*>(ws);
    if (nch > 0 && t.nw > 0) {
      const bool mfma16 = std::is_same<T, bf16>::value && CGTP_LINEAR_BF16_MFMA && t.v8_w && lin->dim_in % 8 == 0 &&
                          lin->dim_out % 8 == 0 && aligned16(x, 16) && aligned16(g, 16);
      if (mfma16)
        hipLaunchKernelGGL(lin_dw_bf16_kernel, dim3(unsigned(nch), unsigned(t.nw)), dim3(kLinThreads), 0, s,
                           static_cast<const bf16*>(x), lin->dim_in, static_cast<const bf16*>(g), lin->dim_out, part,
                           lin->w_numel, B, dw_rows_per_chunk(B), t.wjobs);
      else
        hipLaunchKernelGGL((lin_dw_kernel<T>), dim3(unsigned(nch), unsigned(t.nw)), dim3(kLinThreads), 0, s,
                           static_cast<const T*>(x), lin->dim_in, static_cast<const T*>(g), lin->dim_out, part,
                           lin->w_numel, B, dw_rows_per_chunk(B), t.wjobs);
      CGTP_CHECK_HIP(hipGetLastError());
    }
    hipLaunchKernelGGL((lin_colsum_kernel<T>), dim3(unsigned((lin->w_numel + kLinThreads - 1) / kLinThreads)),
                       dim3(kLinThreads), 0, s, part, static_cast<T*>(dw), nch, lin->w_numel);
    CGTP_CHECK_HIP(hipGetLastError());
  }
}

}  // namespace

cgtp_linear_s* build_linear(const char* irreps_in, const char* irreps_out, cgtp_dtype dtype) {
  if (dtype == CGTP_F64) throw Error{CGTP_ERR_UNSUPPORTED, "linear: fp64 is not supported (fp32, bf16)"};
  if (dtype != CGTP_F32 && dtype != CGTP_BF16) throw Error{CGTP_ERR_INVALID_ARG, "bad dtype"};
  auto lin = std::make_unique<cgtp_linear_s>();
  lin->I = irreps_from_string(irreps_in);
  lin->O = irreps_from_string(irreps_out);
  lin->dtype = dtype;
  int64_t o = 0;
  for (const Irrep& r : lin->I) {
    lin->in_off.push_back(o);
    o += int64_t(r.mul) * (2 * r.l + 1);
  }
  lin->dim_in = o;
  o = 0;
  for (const Irrep& r : lin->O) {
    lin->out_off.push_back(o);
    o += int64_t(r.mul) * (2 * r.l + 1);
  }
  lin->dim_out = o;
  int64_t w = 0;
  for (size_t i = 0; i < lin->I.size(); ++i)
    for (size_t k = 0; k < lin->O.size(); ++k)
      if (lin->I[i].l == lin->O[k].l && lin->I[i].p == lin->O[k].p) {
        lin->paths.push_back({int(i), int(k), lin->I[i].l, lin->I[i].mul, lin->O[k].mul, w});
        w += int64_t(lin->I[i].mul) * lin->O[k].mul;
      }
  lin->w_numel = w;
  if (lin->dim_in > INT32_MAX || lin->dim_out > INT32_MAX || w > INT32_MAX)
    throw Error{CGTP_ERR_UNSUPPORTED, "linear: row or weights too large for 32-bit offsets"};
  return lin.release();
}

void free_linear_tables(const cgtp_linear_s* lin) {
  std::lock_guard<std::mutex> lock(g_lin_mu);
  int cur = 0;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  for (auto it = g_lin_tables.begin(); it != g_lin_tables.end();) {
    if (it->first.first == lin) {
      if (hipSetDevice(it->first.second) == hipSuccess) {
        (void)hipFree(it->second.fjobs);
        (void)hipFree(it->second.fterms);
        (void)hipFree(it->second.xjobs);
        (void)hipFree(it->second.xterms);
        (void)hipFree(it->second.wjobs);
      }
      it = g_lin_tables.erase(it);
    } else {
      ++it;
    }
  }
  if (have) (void)hipSetDevice(cur);
}

void linear_forward_launch(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, void* out,
                           hipStream_t s) {
  if (lin->dtype == CGTP_BF16)
    forward_typed<bf16>(lin, B, x, w, out, s);
  else
    forward_typed<float>(lin, B, x, w, out, s);
}

void linear_backward_launch(const cgtp_linear_s* lin, int64_t B, const void* x, const void* w, const void* g,
                            void* dx, void* dw, void* ws, size_t ws_bytes, hipStream_t s) {
  if (dw && ws_bytes < linear_backward_ws_bytes(lin, B))
    throw Error{CGTP_ERR_WORKSPACE, "linear backward: workspace too small"};
  if (lin->dtype == CGTP_BF16)
    backward_typed<bf16>(lin, B, x, w, g, dx, dw, ws, s);
  else
    backward_typed<float>(lin, B, x, w, g, dx, dw, ws, s);
}

size_t linear_backward_ws_bytes(const cgtp_linear_s* lin, int64_t B) {
  return size_t(dw_chunks(B)) * size_t(lin->w_numel) * sizeof(float);
}

}  // namespace cgtp
