// The radial network's last layer joined to the convolution: per-edge weights
// w[e] = h[e] W2 formed on the matrix cores inside the convolution forward,
// never written to memory.
//
// What is computed: the convolution of conv_impl.hpp (MolSSI e3nn course,
// lesson 06a) with w[e, k] = sum_j h[e, j] W2[j, k], h [E][H] the radial
// network's hidden activations (CSR order) and W2 [H][W] its last layer.
// "E3J: An Efficient and Open-Source Backend for Euclidean Equivariant
// Operations on GPU and TPU", E.4 and F.1: fuse message formation and avoid
// materialising edge-wise intermediates in HBM; xnn, "Run Models on Fused GPU
// Kernels", section "What to expect from fast implementations": radial
// networks above one million edges are recomputed rather than stored.
//
// Forward: one launch per (x block, slot chunk) of the fused forward's
// accumulator layout, a persistent grid of one workgroup per compute unit,
// each with 4 consumer and 4 producer waves walking a contiguous range of the
// receiver schedule. The edges of its receivers go in batches of 16 (32 when
// the block has at most 64 channels) through a two-stage pipeline:
//   producers: the batch's weight tile wt[edges][slots x u] on
//     v_mfma_f32_16x16x4_f32, D[col][edge] = sum_j W2[j][col] h[edge][j]
//     (A = W2 columns, the same for every batch of the launch and kept in
//     registers; B = h), into one of two LDS buffers;
//   consumers: the previous batch, lane groups of u / 4 lanes (4 channels per
//     lane), two edges per group at a time, running the slot's compile-time
//     coefficient pattern with w read from the other buffer.
// A wave's register count is the larger of the two roles, not their sum, and
// the matrix-core work of one batch overlaps the vector-ALU work of the last.
// The edge groups' partial sums are added in a fixed order (lanes of a wave,
// then waves in order) and stored once per receiver. Results are
// deterministic; the sum over a receiver's edges runs in a different order
// than the fused forward's (edge groups of a batch first), which is within
// rounding.
//
// Backward, composed through the workspace: w = h W2 (the linear map's
// kernel), the convolution backward (grad_x, grad_sh, grad_w), then the
// linear map's backward for grad_h = grad_w W2^T and grad_W2 = h^T grad_w.
#include <algorithm>
#include <map>
#include <memory>
#include <mutex>

#include "conv_impl.hpp"
#include "linear.hpp"

namespace cgtp {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

struct RadialArgs {
  ConvArgs a;          // plan tables, graph, x, sh, out, scale (a.w unused)
  const float* h;      // [E][H]
  const float* W2;     // [H][W]
  int H;               // multiple of 4
};

constexpr int kRBudget = conv_budget<float, 4>();  // accumulator entries per channel of a slot chunk
constexpr int kRProd = 4;                          // producer waves (weight tiles on the matrix cores)
constexpr int kRCons = 4;                          // consumer waves (tensor product)
constexpr int kRTab = 64;                          // ints of LDS for the chunk's present-slot table
constexpr int kRRes = 8;                           // tiles per producer wave whose A operands stay in registers

template <int L1, int L>
constexpr int radial_nchunks() { return Chunks<Slots<L1, L>, kRBudget>::NCH; }

template <int L1, int L>
int radial_chunk_slots(int ch) {
  using CK = Chunks<Slots<L1, L>, kRBudget>;
  return CK::arr.begin[ch + 1] - CK::arr.begin[ch];
}

// LDS: the slot table, two weight tiles [edges][slots x u + 4] (double
// buffer), and the consumer waves' partial sums [waves][budget][u] (floats).
size_t radial_lds_bytes(int slots, int U, int edges) {
  const size_t tiles = 2 * size_t(edges) * size_t(slots * U + 4);
  const size_t red = size_t(kRCons) * size_t(kRBudget) * size_t(U);
  return kRTab * sizeof(int) + (tiles + red) * sizeof(float);
}

// The receivers of a workgroup's range, walked batch by batch (a receiver
// without edges is one empty batch, so that its outputs are written).
struct BatchWalk {
  int64_t pos, end, n;
  int32_t base, e1;
  int nb;
  bool valid, last;
  __device__ void enter(const ConvArgs& a, int RE) {
    valid = pos < end;
    if (!valid) return;
    n = a.order[pos];
    base = a.row_ptr[n];
    e1 = n == a.pad ? base : a.row_ptr[n + 1];  // padding edges skipped
    set(RE);
  }
  __device__ void set(int RE) {
    nb = e1 - base < RE ? e1 - base : RE;
    last = base + RE >= e1;
  }
  __device__ void next(const ConvArgs& a, int RE) {
    if (last) {
      ++pos;
      enter(a, RE);
    } else {
      base += RE;
      set(RE);
    }
  }
};

// One launch per (x block, slot chunk); a persistent grid in which workgroup
// w (renumbered so that each XCD takes one contiguous part of the schedule)
// walks receivers [w N / G, (w + 1) N / G) of the receiver schedule.
// Waves 0 .. 3 run the tensor product, waves 4 .. 7 form weight tiles. The
// batches of all the workgroup's receivers go through a two-stage pipeline:
// in step t the producers form the tile of batch t into buffer t mod 2 while
// the consumers run batch t - 1 from the other buffer. Two barriers end each
// step; between them the consumers hand the partial sums of a finished
// receiver to LDS, and after the second the consumer waves add them in wave
// order (accumulator row r by wave r mod 4) and store the receiver's outputs.
//
// Producer tile: D[col][edge] = sum_k W2[k][col] h[edge][k] on
// v_mfma_f32_16x16x4_f32, one 16-column tile of a present slot for one
// 16-edge N tile at a time; lane (i = lane mod 16, q = lane / 16) supplies in
// step st the contraction index k = (H / 4) q + st (A = W2[k][col0 + i],
// B = h[edge i][k]) and holds D[4 q + r][i], stored to
// tile[edge i][slot u + col0 + 4 q + r]. A producer wave's (tile, N tile)
// pairs are the same for every batch: at H = 64 the A operands of its first
// kRRes pairs stay in registers for the whole launch, the others are read per
// batch (the next one requested before the current products run), and the
// next batch's h is requested before the current batch's products run.
template <int L1, int L, int CH>
__global__ __launch_bounds__((kRCons + kRProd) * 64) void conv_fwd_radial_kernel(RadialArgs ra, int NT) {
  using S = Slots<L1, L>;
  using CK = Chunks<S, kRBudget>;
  constexpr int NC = kRCons;
  const ConvArgs& a = ra.a;
  extern __shared__ __attribute__((aligned(16))) float rsm[];
  // [0]: present slots P; [1 + 2 i], [2 + 2 i]: slot index, W2 column; [32 + k]: output offset of slot k
  int* tab = reinterpret_cast<int*>(rsm);
  float* buf = rsm + kRTab;
  const int RE = 16 * NT;
  const BlockDev blk = ldc(a.blocks + a.block);
  const int U = blk.mul;  // 16 .. 256, U / 4 a power of two (checked by the launcher)
  const int LG = U >> 2, NG = NC * 64 / LG;
  const int tid = int(threadIdx.x), lane = tid & 63, wave = conv_wave_id(), li16 = lane & 15, lq = lane >> 4;
  const int gi = tid / LG, c = 4 * (tid - gi * LG);  // consumers: edge group, channels
  const int64_t G = gridDim.x, w = xcd_block();
  BatchWalk walk;
  walk.pos = w * a.N / G;
  walk.end = (w + 1) * a.N / G;
  walk.enter(a, RE);
  const int so = ldc(a.slot_off + a.block);
  const int H = ra.H, Q = H >> 2;
  {
    constexpr int s0 = CK::arr.begin[CH], s1 = CK::arr.begin[CH + 1], NSC = s1 - s0;
    constexpr int acc0 = S::arr.p[s0].acc;
    constexpr int NACC = (s1 < S::NS ? S::arr.p[s1 < S::NS ? s1 : 0].acc : S::NACC) - acc0;
    const int WP = NSC * U + 4;
    const int TS = RE * WP;                 // floats per tile buffer
    float* red = buf + 2 * TS;              // [NC][kRBudget][U]
    int pid[NSC];
#pragma unroll
    for (int k = 0; k < NSC; ++k) pid[k] = ldc(a.slot_paths + so + S::arr.p[s0 + k].src);
    if (tid == NC * 64) {  // the chunk's present slots, for the producers' runtime tile index
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < NSC; ++k)
        if (pid[k] >= 0) {
          tab[1 + 2 * cnt] = k;
          tab[2 + 2 * cnt] = ldc(&a.paths[pid[k]].w_off);
          ++cnt;
        }
      tab[0] = cnt;
#pragma unroll
      for (int k = 0; k < NSC; ++k) tab[kRTab / 2 + k] = pid[k] >= 0 ? ldc(&a.paths[pid[k]].out_off) : -1;
    }
    __syncthreads();
    if (wave >= NC) {
      // ------------------------------------------------------------ producers
      const int pw = wave - NC, tpk = U >> 4, T = tab[0] * tpk;
      const int nt = pw % NT, fs = kRProd / NT;  // this wave's N tile; tile stride
      const int f0 = pw / NT;
      const float* __restrict__ W2 = ra.W2;
      auto load_a = [&](int f, float (&av)[16]) {  // H = 64: k = 16 q + st
        const int i = f / tpk, ct = f - i * tpk;
        const float* __restrict__ w2c = W2 + tab[2 + 2 * i] + 16 * ct + li16 + int64_t(16 * lq) * a.W;
#pragma unroll
        for (int st = 0; st < 16; ++st) av[st] = w2c[int64_t(st) * a.W];
      };
      auto load_b = [&](const BatchWalk& b, float (&bv)[16]) {  // h[edge][16 q .. 16 q + 15], zero past the batch
        const int ed = 16 * nt + li16;
        const bool ok = ed < b.nb;
        const float4* hp = reinterpret_cast<const float4*>(ra.h + int64_t(ok ? b.base + ed : 0) * 64 + 16 * lq);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4 hv = ok ? hp[v] : make_float4(0.f, 0.f, 0.f, 0.f);
          bv[4 * v] = hv.x;
          bv[4 * v + 1] = hv.y;
          bv[4 * v + 2] = hv.z;
          bv[4 * v + 3] = hv.w;
        }
      };
      auto store_d = [&](float* wt, int f, const v4f& d) {
        const int i = f / tpk, ct = f - i * tpk;
        *reinterpret_cast<v4f*>(wt + (16 * nt + li16) * WP + tab[1 + 2 * i] * U + 16 * ct + 4 * lq) = d;
      };
      const int nw = T > f0 ? (T - f0 + fs - 1) / fs : 0;  // this wave's tiles
      float ar[kRRes][16];
      float bn[16];
      if (H == 64) {
        static_for<0, kRRes>([&](auto Rc) {
          constexpr int r = decltype(Rc)::value;
          if (r < nw) load_a(f0 + fs * r, ar[r]);
        });
        if (walk.valid) load_b(walk, bn);
      }
      for (int t = 0;; ++t) {
        const bool have = walk.valid;
        if (have) {
          float* __restrict__ wt = buf + (t & 1) * TS;
          BatchWalk nx = walk;
          nx.next(a, RE);
          if (H == 64) {
            float bb[16];
#pragma unroll
            for (int st = 0; st < 16; ++st) bb[st] = bn[st];
            if (nx.valid) load_b(nx, bn);
            static_for<0, kRRes>([&](auto Rc) {
              constexpr int r = decltype(Rc)::value;
              if (r < nw) {
                v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 16; ++st) d = __builtin_amdgcn_mfma_f32_16x16x4f32(ar[r][st], bb[st], d, 0, 0, 0);
                store_d(wt, f0 + fs * r, d);
              }
            });
            if (nw > kRRes) {
              float an[16];
              load_a(f0 + fs * kRRes, an);
              for (int f = f0 + fs * kRRes; f < T; f += fs) {
                float av[16];
#pragma unroll
                for (int st = 0; st < 16; ++st) av[st] = an[st];
                if (f + fs < T) load_a(f + fs, an);
                v4f d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int st = 0; st < 16; ++st) d = __builtin_amdgcn_mfma_f32_16x16x4f32(av[st], bb[st], d, 0, 0, 0);
                store_d(wt, f, d);
              }
            }
          } else {
            const int ed = 16 * nt + li16;
            const bool ok = ed < walk.nb;
            const float* __restrict__ hr = ra.h + int64_t(ok ? walk.base + ed : 0) * H + Q * lq;
            for (int f = f0; f < T; f += fs) {
              const int i = f / tpk, ct = f - i * tpk;
              const float* __restrict__ w2c = W2 + tab[2 + 2 * i] + 16 * ct + li16 + int64_t(Q * lq) * a.W;
              v4f d = {0.f, 0.f, 0.f, 0.f};
              for (int st = 0; st < Q; ++st)
                d = __builtin_amdgcn_mfma_f32_16x16x4f32(w2c[int64_t(st) * a.W], ok ? hr[st] : 0.f, d, 0, 0, 0);
              store_d(wt, f, d);
            }
          }
          walk = nx;
        }
        __syncthreads();  // A: the tile of this step is formed, the previous one consumed
        __syncthreads();  // B: a finished receiver's partial sums are in LDS
        if (!have) break;
      }
    } else {
      // ------------------------------------------------------------ consumers
      const float* __restrict__ X = static_cast<const float*>(a.x);
      const float* __restrict__ cf = static_cast<const float*>(a.coef);
      int coff[NSC];
#pragma unroll
      for (int k = 0; k < NSC; ++k) coff[k] = pid[k] >= 0 ? ldc(&a.paths[pid[k]].coef_off) : 0;  // absent: discarded
      float acc[NACC][4];
#pragma unroll
      for (int i = 0; i < NACC; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][v] = 0.f;
      __syncthreads();  // step 0: the producers form the first tile
      __syncthreads();
      for (int t = 1; walk.valid; ++t) {
        const float* __restrict__ wt = buf + ((t - 1) & 1) * TS;
        // a group's edges two at a time: both gathers are requested before
        // either product runs
        for (int kk = gi; kk < walk.nb; kk += 2 * NG) {
          const bool two = kk + NG < walk.nb;
          const int k1 = two ? kk + NG : kk;
          const int64_t ea = walk.base + kk, eb = walk.base + k1;
          const int64_t ja = a.src[ea], jb = a.src[eb];
          float xa[2 * L1 + 1][4], xb[2 * L1 + 1][4];
#pragma unroll
          for (int m = 0; m < 2 * L1 + 1; ++m) {
            VecIO<float, 4>::load(X + ja * a.dim_x + blk.x_off + m * U + c, xa[m]);
            VecIO<float, 4>::load(X + jb * a.dim_x + blk.x_off + m * U + c, xb[m]);
          }
          const float* __restrict__ Ya = static_cast<const float*>(a.sh) + ea * a.dim_y;
          const float* __restrict__ Yb = static_cast<const float*>(a.sh) + eb * a.dim_y;
          const float* __restrict__ wra = wt + kk * WP + c;
          const float* __restrict__ wrb = wt + k1 * WP + c;
          float ya[2 * L + 1], yb[2 * L + 1];
          static_for<s0, s1>([&](auto I) {
            constexpr int i = decltype(I)::value;
            constexpr SlotT st = S::arr.p[i];
            constexpr bool first_of_l2 = (i == s0) || (S::arr.p[i > 0 ? i - 1 : 0].l2 != st.l2);
            if constexpr (first_of_l2) {
              const int yo = a.yoff[st.l2];
              const float* __restrict__ ypa = yo >= 0 ? Ya + yo : cf;
              const float* __restrict__ ypb = yo >= 0 ? Yb + yo : cf;
#pragma unroll
              for (int m = 0; m < 2 * st.l2 + 1; ++m) {
                ya[m] = ypa[m];
                yb[m] = ypb[m];
              }
            }
            if (pid[i - s0] >= 0) {  // an absent slot's tile columns are never written
              const v4f wa = *reinterpret_cast<const v4f*>(wra + (i - s0) * U);
              const v4f wb = *reinterpret_cast<const v4f*>(wrb + (i - s0) * U);
              float y2[2 * st.l2 + 1];
              float tt[2 * st.l3 + 1][4];
#pragma unroll
              for (int m = 0; m < 2 * st.l2 + 1; ++m) y2[m] = ya[m];
              fwd_core<L1, st.l2, st.l3, 4, float>(xa, y2, cf + coff[i - s0], tt);
#pragma unroll
              for (int m = 0; m < 2 * st.l3 + 1; ++m)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[st.acc - acc0 + m][v] = fma(wa[v], tt[m][v], acc[st.acc - acc0 + m][v]);
              if (two) {
#pragma unroll
                for (int m = 0; m < 2 * st.l2 + 1; ++m) y2[m] = yb[m];
                fwd_core<L1, st.l2, st.l3, 4, float>(xb, y2, cf + coff[i - s0], tt);
#pragma unroll
                for (int m = 0; m < 2 * st.l3 + 1; ++m)
#pragma unroll
                  for (int v = 0; v < 4; ++v) acc[st.acc - acc0 + m][v] = fma(wb[v], tt[m][v], acc[st.acc - acc0 + m][v]);
              }
            }
          });
        }
        __syncthreads();  // A
        const bool fin = walk.last;
        if (fin) {
          // edge groups of a wave (lanes with equal channels), one accumulator
          // row at a time; then the waves in order
#pragma unroll
          for (int i = 0; i < NACC; ++i) {
            xor_sum_n<4>(acc[i], LG, 64);
            if (lane < LG) *reinterpret_cast<v4f*>(red + (wave * kRBudget + i) * U + c) = v4f{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[i][v] = 0.f;
          }
        }
        __syncthreads();  // B
        if (fin && lane < LG) {  // accumulator row r is summed and stored by consumer wave r mod NC
          float* __restrict__ outn = static_cast<float*>(a.out) + walk.n * a.dim_out;
          const float sc = float(a.scale);
          static_for<s0, s1>([&](auto I) {
            constexpr int i = decltype(I)::value;
            constexpr SlotT st = S::arr.p[i];
            const int oo = tab[kRTab / 2 + (i - s0)];
            if (oo >= 0) {
#pragma unroll
              for (int m = 0; m < 2 * st.l3 + 1; ++m) {
                const int r = st.acc - acc0 + m;
                if (r % NC == wave) {
                  v4f sum = *reinterpret_cast<const v4f*>(red + r * U + c);
#pragma unroll 1
                  for (int q = 1; q < NC; ++q) sum += *reinterpret_cast<const v4f*>(red + (q * kRBudget + r) * U + c);
                  float o[4] = {sc * sum[0], sc * sum[1], sc * sum[2], sc * sum[3]};
                  VecIO<float, 4>::store(outn + oo + m * U + c, o);
                }
              }
            }
          });
        }
        walk.next(a, RE);
      }
    }
  }
}

template <int D, int M, int CH>
void launch_radial(const RadialArgs& ra, int NT, unsigned grid, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((conv_fwd_radial_kernel<D, M, CH>), dim3(grid), dim3((kRCons + kRProd) * 64), lds, s, ra, NT);
}

std::mutex g_rad_mu;
std::map<std::pair<const cgtp_plan_s*, int>, std::unique_ptr<cgtp_linear_s>> g_rad_lin;  // (plan, H) -> h -> w map

// The last layer as a linear map "H x 0e" -> "W x 0e" with W_p = W2 [H][W].
const cgtp_linear_s* hidden_map(const cgtp_plan_s* plan, int H) {
  std::lock_guard<std::mutex> lock(g_rad_mu);
  auto& slot = g_rad_lin[{plan, H}];
  if (!slot) {
    auto lin = std::make_unique<cgtp_linear_s>();
    lin->dtype = CGTP_F32;
    lin->I.push_back(Irrep{H, 0, 1});
    lin->O.push_back(Irrep{int(plan->w_numel), 0, 1});
    lin->in_off.push_back(0);
    lin->out_off.push_back(0);
    lin->paths.push_back(cgtp_linear_s::Path{0, 0, 0, H, int(plan->w_numel), 0});
    lin->dim_in = H;
    lin->dim_out = plan->w_numel;
    lin->w_numel = int64_t(H) * plan->w_numel;
    slot = std::move(lin);
  }
  return slot.get();
}

size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t radial_lds_limit() {
  int dev = 0, v = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  CGTP_CHECK_HIP(hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev));
  return size_t(v);
}

void radial_checks(const cgtp_plan_s* plan, int64_t H) {
  if (plan->dtype != CGTP_F32) throw Error{CGTP_ERR_UNSUPPORTED, "radial convolution: fp32 only"};
  if (plan->collapse || !plan->conv_fused)
    throw Error{CGTP_ERR_UNSUPPORTED, "radial convolution: needs distinct y degrees and uncollapsed outputs"};
  if (H <= 0 || H % 4 != 0 || H > 1024) throw Error{CGTP_ERR_UNSUPPORTED, "radial convolution: hidden width must be a multiple of 4 (<= 1024)"};
  for (const BlockInfo& b : plan->blocks) {
    const int lg = b.mul / 4;
    if (b.mul % 16 != 0 || lg > 64 || (lg & (lg - 1)) != 0)
      throw Error{CGTP_ERR_UNSUPPORTED, "radial convolution: x multiplicities must be 16, 32, 64, 128 or 256"};
  }
}

}  // namespace

void free_radial_maps(const cgtp_plan_s* plan) {
  std::lock_guard<std::mutex> lock(g_rad_mu);
  for (auto it = g_rad_lin.begin(); it != g_rad_lin.end();) {
    if (it->first.first == plan) {
      free_linear_tables(it->second.get());
      it = g_rad_lin.erase(it);
    } else {
      ++it;
    }
  }
}

void conv_forward_radial_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh, const void* h,
                                int64_t H, const void* W2, double scale, void* out, hipStream_t s) {
  radial_checks(plan, H);
  if (g->E == 0) {
    zero_rows(out, g->N * plan->dim_out, dtype_size(plan->dtype), s);
    return;
  }
  const DevTables& t = plan_tables(plan);
  RadialArgs ra{};
  ConvArgs& a = ra.a;
  a.paths = t.paths;
  a.blocks = t.blocks;
  a.coef = t.coef;
  a.slot_paths = t.slot_paths;
  a.slot_off = t.slot_off;
  a.row_ptr = g->row_ptr;
  a.src = g->src;
  a.order = g->order;
  a.N = g->N;
  a.dim_x = int(plan->dim_x);
  a.dim_y = int(plan->dim_y);
  a.dim_out = int(plan->dim_out);
  a.W = int(plan->w_numel);
  a.L = plan->conv_L;
  a.pad = g->pad;
  for (int l = 0; l <= kLmax; ++l) a.yoff[l] = plan->yoff_by_l[l];
  a.x = x;
  a.sh = sh;
  a.out = out;
  a.scale = scale;
  ra.h = static_cast<const float*>(h);
  ra.W2 = static_cast<const float*>(W2);
  ra.H = int(H);
  int dev = 0, cus = 0;
  CGTP_CHECK_HIP(hipGetDevice(&dev));
  CGTP_CHECK_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  // one 8-wave workgroup fits a compute unit (up to 256 registers per lane)
  const unsigned grid = unsigned(std::min<int64_t>(g->N, int64_t(cus)));
  for (size_t b = 0; b < plan->blocks.size(); ++b) {
    a.block = int(b);
    const int l1 = plan->blocks[b].l1, L = plan->conv_L, U = plan->blocks[b].mul;
    bool done = false;
    static_for<0, kLmax + 1>([&](auto I) {
      static_for<0, kLmax + 1>([&](auto J) {
        constexpr int D = decltype(I)::value, M = decltype(J)::value;
        if constexpr (Slots<D, M>::NS > 0) {
          if (!done && l1 == D && L == M) {
            const int NT = U <= 64 ? 2 : 1;  // 32-edge batches for narrow blocks
            static_for<0, radial_nchunks<D, M>()>([&](auto C) {
              constexpr int CH = decltype(C)::value;
              const size_t lds = radial_lds_bytes(radial_chunk_slots<D, M>(CH), U, 16 * NT);
              if (lds > radial_lds_limit())
                throw Error{CGTP_ERR_UNSUPPORTED, "radial convolution: tiles exceed the LDS"};
              launch_radial<D, M, CH>(ra, NT, grid, lds, s);
              CGTP_CHECK_HIP(hipGetLastError());
            });
            done = true;
          }
        }
      });
    });
  }
}

size_t conv_backward_radial_ws_bytes(const cgtp_plan_s* plan, const cgtp_graph_s* g, int64_t H) {
  const size_t ew = align256(size_t(g->E) * size_t(plan->w_numel) * sizeof(float));
  return 2 * ew + align256(conv_backward_ws_bytes(plan, g)) +
         linear_backward_ws_bytes(hidden_map(plan, int(H)), g->E);
}

void conv_backward_radial_launch(cgtp_plan_s* plan, const cgtp_graph_s* g, const void* x, const void* sh,
                                 const void* h, int64_t H, const void* W2, double scale, const void* grad_out,
                                 void* grad_x, void* grad_sh, void* grad_h, void* grad_W2, void* ws, size_t ws_bytes,
                                 hipStream_t s) {
  radial_checks(plan, H);
  const size_t need = conv_backward_radial_ws_bytes(plan, g, H);
  if (!ws || ws_bytes < need)
    throw Error{CGTP_ERR_WORKSPACE, "conv_backward_radial needs " + std::to_string(need) + " workspace bytes"};
  const cgtp_linear_s* lin = hidden_map(plan, int(H));
  const size_t ew = align256(size_t(g->E) * size_t(plan->w_numel) * sizeof(float));
  char* w = static_cast<char*>(ws);
  char* dw = w + ew;
  char* cws = dw + ew;
  char* lws = cws + align256(conv_backward_ws_bytes(plan, g));
  if (g->E > 0) linear_forward_launch(lin, g->E, h, W2, w, s);
  const bool need_w = grad_h || grad_W2;
  conv_backward_launch(plan, g, x, sh, w, scale, grad_out, grad_x, grad_sh, need_w ? dw : nullptr, cws,
                       size_t(lws - cws), s);
  if (need_w) linear_backward_launch(lin, g->E, h, W2, dw, grad_h, grad_W2, lws, ws_bytes - size_t(lws - w), s);
}

}  // namespace cgtp
