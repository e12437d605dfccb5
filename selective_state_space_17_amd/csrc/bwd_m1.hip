// Gradients of the Mamba-1 selective scan for gfx950 (MI355X).
//
// The forward operation is the selective recurrence of "P20 - Mamba", 5 and
// "03 - Modelos de espacio de estados" ("El mecanismo selectivo de Mamba",
// "Discretizacion"): per (b, c, n) and time t
//   a_t = exp(delta_t A[c,n]),  h_t = a_t h_{t-1} + delta_t B_t[n] x_t,
//   y_t = sum_n C_t[n] h_t + D[c] x_t,  out_t = y_t silu(z_t).
// Reverse mode through that loop, for upstream gradients g_t = dL/dout_t and
// dL/dh_{L-1} (dfinal):
//   dy_t = g_t silu(z_t),  dz_t = g_t y_t silu'(z_t)
//   lam_t = C_t dy_t + a_{t+1} lam_{t+1}         (adjoint of h_t)
//   dC_t[n] = sum_c dy_t h_t,   dB_t[n] = sum_c lam_t delta_t x_t
//   ddelta_t = sum_n lam_t (A a_t h_{t-1}) + x_t sum_n lam_t B_t
//   dx_t = D dy_t + delta_t sum_n lam_t B_t
//   dA[c,n] = sum_{b,t} lam_t a_t h_{t-1} delta_t,  dD[c] = sum_{b,t} dy_t x_t
//   dh0 = a_0 lam_0
//
// Mapping.  A block of 4 waves owns 16 channels of one batch row; lane
// (row cl = tid/16, n = tid%16) holds state n of channel c0 + cl (dstate <=
// 16; the other lanes carry zeros).  The reverse walk needs h_{t-1} at every
// step, so:
//   phase A  walks the sequence forward once (the exp and FMA of the
//            forward recurrence only) and writes the state entering every
//            16-step tile to a checkpoint workspace;
//   phase B  walks the tiles backwards; per tile it reloads the checkpoint,
//            recomputes the 16 states and decays into registers, then runs
//            the adjoint recursion over them.
// Per-(t, c) values (delta, delta*x, dy) and per-(t, n) values (B, C) are
// staged in LDS once per tile.  Sums over the 16 states of a channel (y for
// dz, and the two sums that make ddelta and dx) are done by writing each
// lane's 16 per-step products to LDS and reading them back transposed, so
// lane (cl, s) adds the 16 products of step s; sums over the 16 channels of
// a block (dB, dC) go through the same LDS area and are written as one
// partial per block, which a second kernel adds in a fixed order (the result
// does not depend on scheduling).  dA and dD partials per batch row are
// added the same way.
#include "internal.h"

namespace mssm {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
constexpr int kThreads = 256;
constexpr int kCPB = 16;   // channels per block
constexpr int kTT = 16;    // steps per tile (= checkpoint interval)

template <typename T> struct Io;
template <> struct Io<float> {
  __device__ static float get(const void* p, int64_t i) { return static_cast<const float*>(p)[i]; }
  __device__ static void put(void* p, int64_t i, float v) { static_cast<float*>(p)[i] = v; }
};
template <> struct Io<uint16_t> {
  __device__ static float get(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
  __device__ static void put(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(v));   // nearest even
  }
};

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

template <int CTRL> __device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// sum over the 16 lanes of a row, result in every lane
__device__ __forceinline__ float row_sum(float v) {
  v += dpp<0x128>(v);   // row_ror:8
  v += dpp<0x124>(v);   // row_ror:4
  v += dpp<0x122>(v);   // row_ror:2
  v += dpp<0x121>(v);   // row_ror:1
  return v;
}

// Position of (row cl, state n, step s) in a 16x16x16 fp32 LDS area.  Lane
// (cl, n) writes its 16 steps as four 16-byte stores; the rotation of n by
// the row and the xor of the step by the n group make both transposed reads
// -- lane (cl, s) over n, and thread (s, n) over cl -- hit 64 distinct banks.
__device__ __forceinline__ int qpos(int cl, int n, int s) {
  const int m = (n + cl) & 15;
  return cl * 256 + m * 16 + (s ^ ((m >> 2) << 2));
}

struct BwdParams {
  const void* x;
  const void* delta;
  const void* B;
  const void* C;
  const void* z;       // nullable
  const void* dout;
  const float* A;
  const float* D;      // nullable
  const float* h0;     // nullable
  const float* dfinal; // nullable
  void* dx;
  void* ddelta;
  void* dz;            // written iff z != nullptr
  float* dh0;          // nullable
  float* ckpt;         // [batch][ntiles][ncb*16][16]
  float* partB;        // [ncb][batch][L][16]
  float* partC;        // [ncb][batch][L][16]
  float* wsA;          // [batch][ncb*16][16]
  float* wsD;          // [batch][ncb*16]
  int64_t batch, L, dim, N;
  int ntiles, ncb;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void scan_bwd_kernel(BwdParams p) {
  using io = Io<T>;
  __shared__ float4 TC[kTT][kCPB];   // {delta, delta*x, dy, 0} per (step, channel)
  __shared__ float2 BC[kTT][16];     // {B, C} per (step, state)
  __shared__ __attribute__((aligned(16))) float Q1[16 * 16 * 16];  // dy*h (dC) / transposes / phase A tiles
  __shared__ __attribute__((aligned(16))) float Q2[16 * 16 * 16];  // lam*delta*x (dB) / transposes

  const int tid = threadIdx.x;
  const int cl = tid >> 4;          // compute: channel row
  const int n = tid & 15;           // compute: state
  const int cb = static_cast<int>(blockIdx.x % static_cast<unsigned>(p.ncb));
  const int64_t b = blockIdx.x / static_cast<unsigned>(p.ncb);
  const int64_t c0 = static_cast<int64_t>(cb) * kCPB;
  const int64_t c = c0 + cl;
  const int64_t L = p.L, dim = p.dim, N = p.N;
  const bool lane_ok = c < dim && n < N;
  const int64_t D16 = static_cast<int64_t>(p.ncb) * kCPB;

  const float Av = lane_ok ? p.A[c * N + n] : 0.f;
  const float A2 = Av * kLog2e;
  float* ck = p.ckpt + (b * p.ntiles * D16 + c) * 16 + n;   // + k * D16 * 16

  // -------------------------------------------------------------- phase A
  {
    float4* TCa = reinterpret_cast<float4*>(Q1);        // [2][16][16]
    float2* BCa = reinterpret_cast<float2*>(Q1 + 2048);  // [2][16][16]
    const int ss = tid >> 4, sc = tid & 15;              // staging: step, channel / state
    float h = (lane_ok && p.h0 != nullptr) ? p.h0[(b * dim + c) * N + n] : 0.f;
    float rd = 0.f, rx = 0.f, rb = 0.f;
    auto issue = [&](int k) {
      const int64_t t = static_cast<int64_t>(k) * kTT + ss;
      const int64_t cc = c0 + sc;
      const bool ok = t < L && cc < dim;
      rd = ok ? io::get(p.delta, (b * L + t) * dim + cc) : 0.f;
      rx = ok ? io::get(p.x, (b * L + t) * dim + cc) : 0.f;
      rb = (t < L && sc < N) ? io::get(p.B, (b * L + t) * N + sc) : 0.f;
    };
    if (p.ntiles > 1) issue(0);
    for (int k = 0; k + 1 < p.ntiles; ++k) {
      const int buf = k & 1;
      TCa[buf * 256 + ss * 16 + sc] = float4{rd, rd * rx, 0.f, 0.f};
      BCa[buf * 256 + ss * 16 + sc] = float2{rb, 0.f};
      if (lane_ok) ck[static_cast<int64_t>(k) * D16 * 16] = h;
      __syncthreads();
      if (k + 2 < p.ntiles) issue(k + 1);
#pragma unroll
      for (int s = 0; s < kTT; ++s) {
        const float4 q = TCa[buf * 256 + s * 16 + cl];
        const float bv = BCa[buf * 256 + s * 16 + n].x;
        h = __builtin_fmaf(exp2_hw(q.x * A2), h, q.y * bv);
      }
    }
    if (lane_ok && p.ntiles > 0) ck[static_cast<int64_t>(p.ntiles - 1) * D16 * 16] = h;
    __syncthreads();   // orders the checkpoint stores before phase B's loads; frees Q1
  }

  // -------------------------------------------------------------- phase B
  // staging / finishing role: channel fc = tid/16 (= cl), step fs = tid%16 (= n)
  const int fs = n;
  const float Dc = (c < dim && p.D != nullptr) ? p.D[c] : 0.f;
  float lam = (lane_ok && p.dfinal != nullptr) ? p.dfinal[(b * dim + c) * N + n] : 0.f;
  float dAacc = 0.f, dDacc = 0.f;
  float rdl = 0.f, rx = 0.f, rg = 0.f, rz = 0.f, rb = 0.f, rc = 0.f, rh = 0.f;
  const int bs = tid >> 4, bn = tid & 15;   // B/C staging: step, state
  auto issue = [&](int k) {
    const int64_t t = static_cast<int64_t>(k) * kTT + fs;
    const bool ok = t < L && c < dim;
    const int64_t i = (b * L + t) * dim + c;
    rdl = ok ? io::get(p.delta, i) : 0.f;
    rx = ok ? io::get(p.x, i) : 0.f;
    rg = ok ? io::get(p.dout, i) : 0.f;
    rz = (ok && p.z != nullptr) ? io::get(p.z, i) : 0.f;
    const int64_t tb = static_cast<int64_t>(k) * kTT + bs;
    const bool okb = tb < L && bn < N;
    rb = okb ? io::get(p.B, (b * L + tb) * N + bn) : 0.f;
    rc = okb ? io::get(p.C, (b * L + tb) * N + bn) : 0.f;
    rh = lane_ok ? ck[static_cast<int64_t>(k) * D16 * 16] : 0.f;
  };

  if (p.ntiles > 0) issue(p.ntiles - 1);
  for (int k = p.ntiles - 1; k >= 0; --k) {
    const int64_t t0 = static_cast<int64_t>(k) * kTT;
    const int64_t tf = t0 + fs;
    const bool fvalid = tf < L && c < dim;
    // ---- stage: this thread's (step fs, channel cl) values stay in registers for the finish
    const float dl = rdl, u = rx, du = rdl * rx;
    float dy = rg, sdz = 0.f;
    if (p.z != nullptr) {
      const float sg = __builtin_amdgcn_rcpf(1.f + exp2_hw(-rz * kLog2e));
      dy = rg * rz * sg;
      sdz = rg * sg * __builtin_fmaf(rz, 1.f - sg, 1.f);
    }
    TC[fs][cl] = float4{dl, du, dy, 0.f};
    BC[bs][bn] = float2{rb, rc};
    float h = rh;            // state entering the tile
    const float hin = rh;    // (rh is reloaded for the next tile below)
    __syncthreads();
    if (k > 0) issue(k - 1);

    // ---- recompute the tile's states and decays
    float hs[kTT], av[kTT], pr[kTT], q1[kTT];
#pragma unroll
    for (int s = 0; s < kTT; ++s) {
      const float4 q = TC[s][cl];
      const float2 bc = BC[s][n];
      av[s] = exp2_hw(q.x * A2);
      h = __builtin_fmaf(av[s], h, q.y * bc.x);
      hs[s] = h;
      pr[s] = bc.y * h;      // C h: readout term of y
      q1[s] = q.z * h;       // dy h: dC term
    }
    // Transposes go through this wave's own rows of Q1/Q2 (no other wave
    // touches them before the barrier below); a wave's LDS accesses run in
    // order, so a row is rewritten only after it has been read back.
    auto park = [&](float* area, const float (&v)[kTT]) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(&area[qpos(cl, n, 4 * i)]) = float4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      __builtin_amdgcn_wave_barrier();
    };
    // lane (cl, fs) adds the 16 products of step fs; rows are visited in
    // stored order, so the addresses are four bases plus constant offsets
    auto fetch = [&](const float* area) {
      float r[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float* base = area + cl * 256 + g * 64 + (fs ^ (g << 2));
#pragma unroll
        for (int j = 0; j < 4; ++j) r[4 * g + j] = base[16 * j];
      }
      __builtin_amdgcn_wave_barrier();
      return ((r[0] + r[1]) + (r[2] + r[3]) + ((r[4] + r[5]) + (r[6] + r[7]))) +
             ((r[8] + r[9]) + (r[10] + r[11]) + ((r[12] + r[13]) + (r[14] + r[15])));
    };
    park(Q2, pr);
    const float y = __builtin_fmaf(Dc, u, fetch(Q2));
    park(Q1, q1);            // stays for the channel sums
    const int64_t fi = (b * L + tf) * dim + c;
    if (p.z != nullptr && fvalid) io::put(p.dz, fi, sdz * y);

    // ---- adjoint recursion over the tile, last step first.  Operands are
    // read two steps ahead; the scheduling barrier per step keeps the compiler
    // from hoisting all 16 steps' operands (80 registers) to the loop head.
    float q2[kTT], r1[kTT], r2[kTT];
    float4 qa = TC[kTT - 1][cl], qb = TC[kTT - 2][cl];
    float2 ba = BC[kTT - 1][n], bb = BC[kTT - 2][n];
#pragma unroll
    for (int s = kTT - 1; s >= 0; --s) {
      const float4 q = qa;
      const float2 bc = ba;
      qa = qb;
      ba = bb;
      if (s >= 2) {
        qb = TC[s - 2][cl];
        bb = BC[s - 2][n];
      }
      lam = __builtin_fmaf(bc.y, q.z, lam);          // + C dy
      q2[s] = lam * q.y;                              // lam delta x
      r2[s] = lam * bc.x;                             // lam B
      lam *= av[s];                                   // a_t lam_t
      const float t1 = lam * (s > 0 ? hs[s - 1] : hin);   // lam a_t h_{t-1}
      dAacc = __builtin_fmaf(t1, q.x, dAacc);
      r1[s] = t1 * Av;
      // materialise this step's results here (otherwise the compiler sinks
      // the q2 and dA updates past the loop and keeps their operands alive)
      __asm__ volatile("" : "+v"(dAacc), "+v"(q2[s]), "+v"(r1[s]), "+v"(r2[s]));
      __builtin_amdgcn_sched_barrier(0);
    }
    park(Q2, r1);
    const float s1 = fetch(Q2);
    park(Q2, r2);
    const float s2 = fetch(Q2);
    if (fvalid) {
      io::put(p.ddelta, fi, __builtin_fmaf(u, s2, s1));
      io::put(p.dx, fi, __builtin_fmaf(dl, s2, Dc * dy));
    }
    dDacc = __builtin_fmaf(dy, u, dDacc);
    park(Q2, q2);
    __syncthreads();

    // ---- channel sums of this block: thread (step bs, state bn)
    {
      float sb = 0.f, sc = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc += Q1[qpos(r, bn, bs)];
        sb += Q2[qpos(r, bn, bs)];
      }
      const int64_t t = t0 + bs;
      if (t < L) {
        const int64_t o = ((static_cast<int64_t>(cb) * p.batch + b) * L + t) * 16 + bn;
        p.partB[o] = sb;
        p.partC[o] = sc;
      }
    }
    __syncthreads();   // Q1/Q2/TC/BC are rewritten by the next tile
  }

  if (lane_ok && p.dh0 != nullptr) p.dh0[(b * dim + c) * N + n] = lam;
  p.wsA[(b * D16 + c) * 16 + n] = dAacc;   // zero for padded lanes
  const float dDrow = row_sum(dDacc);
  if (n == 0) p.wsD[b * D16 + c] = dDrow;
}

// dB, dC: sum of the per-block partials, in block order
__global__ __launch_bounds__(256) void bwd_reduce_bc(const float* partB, const float* partC, float* dB, float* dC,
                                                     int64_t batch, int64_t L, int64_t N, int ncb) {
  const int64_t rows = batch * L;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (row, n16)
  if (i >= rows * 16) return;
  const int64_t row = i >> 4;
  const int nn = static_cast<int>(i & 15);
  if (nn >= N) return;
  float sb = 0.f, sc = 0.f;
  for (int k = 0; k < ncb; ++k) {
    sb += partB[k * rows * 16 + i];
    sc += partC[k * rows * 16 + i];
  }
  dB[row * N + nn] = sb;
  dC[row * N + nn] = sc;
}

// dA, dD: sum over the batch rows, in order
__global__ __launch_bounds__(256) void bwd_reduce_ad(const float* wsA, const float* wsD, float* dA, float* dD,
                                                     int64_t batch, int64_t dim, int64_t N, int ncb) {
  const int64_t D16 = static_cast<int64_t>(ncb) * 16;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;   // (c, n16)
  if (i >= dim * 16) return;
  const int64_t cc = i >> 4;
  const int nn = static_cast<int>(i & 15);
  if (nn < N) {
    float s = 0.f;
    for (int64_t bb = 0; bb < batch; ++bb) s += wsA[(bb * D16 + cc) * 16 + nn];
    dA[cc * N + nn] = s;
  }
  if (nn == 0 && dD != nullptr) {
    float s = 0.f;
    for (int64_t bb = 0; bb < batch; ++bb) s += wsD[bb * D16 + cc];
    dD[cc] = s;
  }
}

struct Layout {
  size_t ckpt, partB, partC, wsA, wsD, total;
};
size_t align256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }
Layout layout(int64_t batch, int64_t L, int64_t dim) {
  const int64_t ncb = (dim + kCPB - 1) / kCPB, D16 = ncb * kCPB, nt = (L + kTT - 1) / kTT;
  Layout l{};
  size_t off = 0;
  l.ckpt = off;  off += align256(sizeof(float) * static_cast<size_t>(batch * nt * D16 * 16));
  l.partB = off; off += align256(sizeof(float) * static_cast<size_t>(ncb * batch * L * 16));
  l.partC = off; off += align256(sizeof(float) * static_cast<size_t>(ncb * batch * L * 16));
  l.wsA = off;   off += align256(sizeof(float) * static_cast<size_t>(batch * D16 * 16));
  l.wsD = off;   off += align256(sizeof(float) * static_cast<size_t>(batch * D16));
  l.total = off;
  return l;
}

}  // namespace

size_t scan_bwd_workspace_bytes(int64_t batch, int64_t L, int64_t dim) { return layout(batch, L, dim).total; }

int64_t scan_bwd_grid_blocks(int64_t batch, int64_t dim) { return batch * ((dim + kCPB - 1) / kCPB); }

hipError_t scan_bwd_launch(const ScanBwdArgs& a, hipStream_t stream) {
  const int64_t ncb = (a.dim + kCPB - 1) / kCPB;
  const Layout l = layout(a.batch, a.L, a.dim);
  char* ws = static_cast<char*>(a.workspace);
  BwdParams p{};
  p.x = a.x; p.delta = a.delta; p.B = a.B; p.C = a.C; p.z = a.z; p.dout = a.dout;
  p.A = a.A; p.D = a.D; p.h0 = a.h0; p.dfinal = a.dfinal;
  p.dx = a.dx; p.ddelta = a.ddelta; p.dz = a.dz; p.dh0 = a.dh0;
  p.ckpt = reinterpret_cast<float*>(ws + l.ckpt);
  p.partB = reinterpret_cast<float*>(ws + l.partB);
  p.partC = reinterpret_cast<float*>(ws + l.partC);
  p.wsA = reinterpret_cast<float*>(ws + l.wsA);
  p.wsD = reinterpret_cast<float*>(ws + l.wsD);
  p.batch = a.batch; p.L = a.L; p.dim = a.dim; p.N = a.N;
  p.ntiles = static_cast<int>((a.L + kTT - 1) / kTT);
  p.ncb = static_cast<int>(ncb);
  if (a.batch > 0) {
    const dim3 grid(static_cast<unsigned>(ncb * a.batch));
    if (a.io == 1)
      hipLaunchKernelGGL(scan_bwd_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, p);
    else
      hipLaunchKernelGGL(scan_bwd_kernel<float>, grid, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nbc = (a.batch * a.L * 16 + 255) / 256;
    if (nbc > 0) {
      hipLaunchKernelGGL(bwd_reduce_bc, dim3(static_cast<unsigned>(nbc)), dim3(256), 0, stream, p.partB, p.partC,
                         a.dB, a.dC, a.batch, a.L, a.N, p.ncb);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  const int64_t nad = (a.dim * 16 + 255) / 256;
  hipLaunchKernelGGL(bwd_reduce_ad, dim3(static_cast<unsigned>(nad)), dim3(256), 0, stream, p.wsA, p.wsD, a.dA, a.dD,
                     a.batch, a.dim, a.N, p.ncb);
  return hipGetLastError();
}

}  // namespace mssm
