// Non-causal linear attention for bf16 inputs on gfx950 (MI355X).
//
// Method: "Transformers are RNNs" (Katharopoulos et al., 2020), translated page
// "線性變換器", §3.2 eq.(5)-(6): with S = sum_j phi(k_j) v_j^T and
// z = sum_j phi(k_j) over the whole sequence, o_i = phi(q_i)^T S / phi(q_i)^T z.
// S and z are computed once per (batch, head) and reused by every query.
//
// Three launches, each streaming its operands from HBM once:
//   nc_state_kernel   one workgroup per block of tokens of a head computes the
//                     block's share of S and z (float32) from K and V with
//                     16x16x32 bf16 MFMA tiles; phi(K) is split into a bf16
//                     head and tail so the sum keeps float32-level error.
//   nc_reduce_kernel  sums the block shares of each head in block order (a
//                     fixed order, so results are bitwise repeatable).
//   nc_apply_kernel   every wavefront streams its own rows of Q: phi(Q) times
//                     S (S^T held in registers as bf16 B operands) and times z
//                     (a bf16 head and tail), then o = num / den, stored as bf16.
#include <map>
#include <mutex>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"

namespace la {
namespace nc {

constexpr int NT = 256;  // threads per workgroup (4 wavefronts)
constexpr int CH = 64;   // tokens per chunk of the state kernel

template <int D, int M>
struct G {
  static constexpr int TD = D / 16, TM = M / 16;
  static constexpr int WPT = 4 / TD;    // waves sharing a d-tile of S
  static constexpr int TMW = TM / WPT;  // m-tiles of S per wave
  static constexpr int UK = D / 8;      // 16-byte units per K row
  static constexpr int UV = M / 8;      // 16-byte units per V row
  static constexpr int KV = CH * UK / NT > 0 ? CH * UK / NT : 1;  // K units per thread per chunk
  static constexpr int VV = CH * UV / NT > 0 ? CH * UV / NT : 1;  // V units per thread per chunk
  static constexpr int QV = D / 32;     // d-slabs of a query row
  static constexpr int SZ = D * M + D;  // floats of one (S, z) record
};

template <int D, int M>
struct alignas(16) StateSmem {
  bf16_t Kh[2][CH * D];  // phi(K) head, double-buffered, row-major swizzled
  bf16_t Kl[2][CH * D];  // phi(K) tail
  bf16_t V[2][CH * M];   // V
};

// ----------------------------------------------------------------------------
// Block shares: for slot = bh * nblk + blk,
//   partS + slot * sS = sum_{j in blk} phi(k_j) v_j^T  ([D][M]),
//   partz + slot * sz = sum_{j in blk} phi(k_j)        ([D]).
// Grid: BH * nblk workgroups, blockIdx.x = bh * nblk + blk.
template <int D, int M>
__global__ __launch_bounds__(NT) void nc_state_kernel(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                      int N, int tblk, int nblk, float* __restrict__ partS,
                                                      float* __restrict__ partz, int sS, int sz) {
  using GG = G<D, M>;
  __shared__ StateSmem<D, M> sm;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const int ntok = t1 - t0;
  const int nch2 = (ntok + 2 * CH - 1) / (2 * CH);  // chunk pairs
  const bf16_t* kh = k + ((size_t)bh * N + t0) * D;
  const bf16_t* vh = v + ((size_t)bh * N + t0) * M;

  // Register staging of a chunk: thread unit p = tid + NT * i is (row p / U, unit p % U).
  u32x4 rk[2][GG::KV], rv[2][GG::VV];
  auto load_chunk = [&](int c, u32x4* dk, u32x4* dv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < GG::KV; ++i) {
      const int p = tid + NT * i, row = c * CH + p / GG::UK, cu = p % GG::UK;
      dk[i] = (p < CH * GG::UK && row < ntok) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kh + (size_t)row * D + cu * 8))
                                               : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < GG::VV; ++i) {
      const int p = tid + NT * i, row = c * CH + p / GG::UV, cu = p % GG::UV;
      dv[i] = (p < CH * GG::UV && row < ntok) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vh + (size_t)row * M + cu * 8))
                                               : u32x4{0u, 0u, 0u, 0u};
    }
  };
  load_chunk(0, rk[0], rv[0]);
  load_chunk(1, rk[1], rv[1]);

  f32x4 S[GG::TMW], Z{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) S[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int td = w % GG::TD;
  const bf16x8 ones = ones8();

  for (int c2 = 0; c2 < nch2; ++c2) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 2 * c2 + j;
      // Stage chunk c into buffer j: phi(K) head and tail, V as loaded.
#pragma unroll
      for (int i = 0; i < GG::KV; ++i) {
        const int p = tid + NT * i, row = p / GG::UK, cu = p % GG::UK;
        if (p < CH * GG::UK) {
          u32x4 hv, lv;
          phi_split8(rk[j][i], c * CH + row < ntok, hv, lv);
          unit16<GG::UK>(sm.Kh[j], row, cu * 8) = hv;
          unit16<GG::UK>(sm.Kl[j], row, cu * 8) = lv;
        }
      }
#pragma unroll
      for (int i = 0; i < GG::VV; ++i) {
        const int p = tid + NT * i, row = p / GG::UV, cu = p % GG::UV;
        if (p < CH * GG::UV) unit16<GG::UV>(sm.V[j], row, cu * 8) = rv[j][i];
      }
      load_chunk(c + 2, rk[j], rv[j]);
      // One barrier per chunk: buffer j is rewritten two chunks later, after
      // every wave has passed the next chunk's barrier.
      __syncthreads();
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) {
        const bf16x8 ah = jfrag<GG::UK>(sm.Kh[j], 32 * s, 16 * td, g, n);
        const bf16x8 al = jfrag<GG::UK>(sm.Kl[j], 32 * s, 16 * td, g, n);
#pragma unroll
        for (int u = 0; u < GG::TMW; ++u) {
          const int tm = w / GG::TD + GG::WPT * u;
          const bf16x8 bv = jfrag<GG::UV>(sm.V[j], 32 * s, 16 * tm, g, n);
          S[u] = mma(ah, bv, S[u]);
          S[u] = mma(al, bv, S[u]);
        }
        // every wave forms z (no branch around the MFMAs); waves w < TD store it
        Z = mma(ah, ones, Z);
        Z = mma(al, ones, Z);
      }
    }
  }

  float* dst = partS + ((size_t)bh * nblk + blk) * sS;
#pragma unroll
  for (int u = 0; u < GG::TMW; ++u) {
    const int tm = w / GG::TD + GG::WPT * u;
#pragma unroll
    for (int r = 0; r < 4; ++r) dst[(16 * td + 4 * g + r) * M + 16 * tm + n] = S[u][r];
  }
  if (w < GG::TD && n == 0) {
    float* dz = partz + ((size_t)bh * nblk + blk) * sz;
#pragma unroll
    for (int r = 0; r < 4; ++r) dz[16 * w + 4 * g + r] = Z[r];
  }
}

// ----------------------------------------------------------------------------
// tot[bh] = sum over blk (in order) of part[bh][blk].  Grid: BH * parts; each
// thread owns four consecutive floats of the record.
template <int D, int M>
__global__ __launch_bounds__(NT) void nc_reduce_kernel(const float* __restrict__ part, int nblk, int parts,
                                                       float* __restrict__ tot) {
  using GG = G<D, M>;
  const int bh = blockIdx.x / parts;
  const int e = ((blockIdx.x % parts) * NT + threadIdx.x) * 4;
  if (e >= GG::SZ) return;
  const float* src = part + (size_t)bh * nblk * GG::SZ + e;
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  int b = 0;
  for (; b + 8 <= nblk; b += 8) {
    f32x4 x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = *reinterpret_cast<const f32x4*>(src + (size_t)(b + i) * GG::SZ);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc += x[i];
  }
  for (; b < nblk; ++b) acc += *reinterpret_cast<const f32x4*>(src + (size_t)b * GG::SZ);
  *reinterpret_cast<f32x4*>(tot + (size_t)bh * GG::SZ + e) = acc;
}

// ----------------------------------------------------------------------------
// o = phi(Q) S / phi(Q) z for a block of rows.  Grid: BH * nblk, blockIdx.x =
// bh * nblk + blk.  Wave w handles rows t0 + 64 c + 16 w + (0..15) of every
// 64-row chunk c of the block; after the state is staged the waves never
// synchronise again.
template <int D, int M>
__global__ __launch_bounds__(NT) void nc_apply_kernel(const bf16_t* __restrict__ q, bf16_t* __restrict__ o, int N,
                                                      int tblk, int nblk, const float* __restrict__ tot) {
  using GG = G<D, M>;
  constexpr int PF = 2;  // chunks of queries in flight per wave (2 keeps 120 VGPRs: more resident waves beat deeper queues)
  __shared__ __attribute__((aligned(16))) bf16_t St[M * D];  // S^T [m][d] in bf16, swizzled
  __shared__ __attribute__((aligned(16))) float Zs[D];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int t0 = blk * tblk, t1 = min(N, t0 + tblk);
  const int ntok = t1 - t0;
  const int nchp = (ntok + CH * PF - 1) / (CH * PF);  // groups of PF chunks
  const bf16_t* qh = q + ((size_t)bh * N + t0) * D;
  bf16_t* oh = o + ((size_t)bh * N + t0) * M;

  // Query rows of chunk c for this lane: row 64c + 16w + n, slab s columns 32s + 8g .. +7.
  u32x4 raw[PF][GG::QV];
  auto load_q = [&](int c, u32x4* dq) __attribute__((always_inline)) {
    const int row = CH * c + 16 * w + n;
#pragma unroll
    for (int s = 0; s < GG::QV; ++s)
      dq[s] = row < ntok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 32 * s + 8 * g))
                         : u32x4{0u, 0u, 0u, 0u};
  };
#pragma unroll
  for (int j = 0; j < PF; ++j) load_q(j, raw[j]);

  // Stage S^T (bf16) and z.
  const float* Sh = tot + (size_t)bh * GG::SZ;
  for (int e4 = tid; e4 < D * M / 4; e4 += NT) {
    const int d = e4 / (M / 4), m0 = 4 * (e4 % (M / 4));
    const f32x4 x = *reinterpret_cast<const f32x4*>(Sh + (size_t)d * M + m0);
#pragma unroll
    for (int i = 0; i < 4; ++i) St[swz<GG::UK>(m0 + i, d)] = (bf16_t)(cvt_pk(x[i], 0.f) & 0xffffu);
  }
  if (tid < D) Zs[tid] = Sh[D * M + tid];
  __syncthreads();

  // B operands held for the whole block: column n of m-tile tm is m = TM n + tm,
  // so a lane's outputs are TM consecutive columns.
  bf16x8 bs[GG::QV][GG::TM], zh[GG::QV], zl[GG::QV];
#pragma unroll
  for (int s = 0; s < GG::QV; ++s) {
#pragma unroll
    for (int tm = 0; tm < GG::TM; ++tm) bs[s][tm] = as_bf16x8(unit16<GG::UK>(St, GG::TM * n + tm, 32 * s + 8 * g));
    const f32x4 za = *reinterpret_cast<const f32x4*>(&Zs[32 * s + 8 * g]);
    const f32x4 zb = *reinterpret_cast<const f32x4*>(&Zs[32 * s + 8 * g + 4]);
    u32x4 h, l;
    h[0] = cvt_pk(za[0], za[1]);
    h[1] = cvt_pk(za[2], za[3]);
    h[2] = cvt_pk(zb[0], zb[1]);
    h[3] = cvt_pk(zb[2], zb[3]);
    l[0] = cvt_pk(za[0] - lo_of(h[0]), za[1] - hi_of(h[0]));
    l[1] = cvt_pk(za[2] - lo_of(h[1]), za[3] - hi_of(h[1]));
    l[2] = cvt_pk(zb[0] - lo_of(h[2]), zb[1] - hi_of(h[2]));
    l[3] = cvt_pk(zb[2] - lo_of(h[3]), zb[3] - hi_of(h[3]));
    zh[s] = as_bf16x8(h);
    zl[s] = as_bf16x8(l);
  }

  for (int cp = 0; cp < nchp; ++cp) {
#pragma unroll
    for (int j = 0; j < PF; ++j) {
      const int c = PF * cp + j;
      bf16x8 qf[GG::QV];
#pragma unroll
      for (int s = 0; s < GG::QV; ++s) {
        u32x4 pk;
#pragma unroll
        for (int h = 0; h < 4; ++h) pk[h] = cvt_pk(phi(lo_of(raw[j][s][h])), phi(hi_of(raw[j][s][h])));
        qf[s] = as_bf16x8(pk);
      }
      load_q(c + PF, raw[j]);
      f32x4 num[GG::TM], den{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tm = 0; tm < GG::TM; ++tm) num[tm] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < GG::QV; ++s) {
#pragma unroll
        for (int tm = 0; tm < GG::TM; ++tm) num[tm] = mma(qf[s], bs[s][tm], num[tm]);
        den = mma(qf[s], zh[s], den);
        den = mma(qf[s], zl[s], den);
      }
      // lane (n, g) holds rows 16w + 4g + r of the chunk, columns TM n .. TM n + TM - 1
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = CH * c + 16 * w + 4 * g + r;
        const float inv = __builtin_amdgcn_rcpf(den[r]);
        uint32_t pk[GG::TM / 2];
#pragma unroll
        for (int h = 0; h < GG::TM / 2; ++h) pk[h] = cvt_pk(num[2 * h][r] * inv, num[2 * h + 1][r] * inv);
        bf16_t* dst = oh + (size_t)row * M + GG::TM * n;
        if (row < ntok) {
          if constexpr (GG::TM == 4)
            *reinterpret_cast<u32x2*>(dst) = u32x2{pk[0], pk[1]};
          else
            *reinterpret_cast<uint32_t*>(dst) = pk[0];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Host side.

// Workgroups of `kernel` resident at once on the current device (compute units
// times occupancy), cached per device and kernel.  Without a device the answer
// is 256, so sizes stay defined on hosts with no GPU.
static int resident_wgs(const void* kernel) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, kernel);
  const auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, NT, 0) != hipSuccess || per <= 0) per = 1;
  return cache[key] = cus * per;
}

// Tokens per block so that the BH * nblk workgroups of a kernel fill its
// resident slots about once (whole waves of workgroups, no partial last wave);
// blocks hold whole multiples of `quantum` tokens.
static int block_tokens(int BH, int N, int slots, int quantum) {
  const int per_head = BH >= slots ? 1 : slots / BH;
  int tb = (N + per_head - 1) / per_head;
  tb = (tb + quantum - 1) / quantum * quantum;
  return tb < quantum ? quantum : tb;
}

template <int D, int M>
struct Plan {
  int ts, ns;  // state kernel: tokens per block, blocks per head
  int ta, na;  // apply kernel
  Plan(int BH, int N) {
    ts = block_tokens(BH, N, resident_wgs((const void*)nc_state_kernel<D, M>), 2 * CH);
    ns = (N + ts - 1) / ts;
    ta = block_tokens(BH, N, resident_wgs((const void*)nc_apply_kernel<D, M>), CH);
    na = (N + ta - 1) / ta;
  }
};

template <int D, int M>
static size_t ws_bytes(int BH, int N) {
  const Plan<D, M> p(BH, N);
  return (size_t)BH * (size_t)(p.ns + 1) * G<D, M>::SZ * sizeof(float);
}

template <int D, int M>
static hipError_t impl(const void* q, const void* k, const void* v, void* o, int BH, int N, void* ws,
                       hipStream_t stream) {
  using GG = G<D, M>;
  const Plan<D, M> p(BH, N);
  float* part = (float*)ws;
  float* tot = part + (size_t)BH * p.ns * GG::SZ;
  const dim3 block(NT);
  hipLaunchKernelGGL((nc_state_kernel<D, M>), dim3((unsigned)p.ns * (unsigned)BH), block, 0, stream,
                     (const bf16_t*)k, (const bf16_t*)v, N, p.ts, p.ns, part, part + D * M, GG::SZ, GG::SZ);
  if (p.ns > 1) {
    const int parts = (GG::SZ / 4 + NT - 1) / NT;
    hipLaunchKernelGGL((nc_reduce_kernel<D, M>), dim3((unsigned)(parts * BH)), block, 0, stream, part, p.ns, parts,
                       tot);
  } else {
    tot = part;
  }
  hipLaunchKernelGGL((nc_apply_kernel<D, M>), dim3((unsigned)p.na * (unsigned)BH), block, 0, stream,
                     (const bf16_t*)q, (bf16_t*)o, N, p.ta, p.na, tot);
  return hipGetLastError();
}

}  // namespace nc

size_t noncausal_bf16_ws_bytes(int BH, int N, int D, int M) {
  if (BH <= 0 || N <= 0) return 0;
  switch (D * 100 + M) {
    case 3232: return nc::ws_bytes<32, 32>(BH, N);
    case 3264: return nc::ws_bytes<32, 64>(BH, N);
    case 6432: return nc::ws_bytes<64, 32>(BH, N);
    case 6464: return nc::ws_bytes<64, 64>(BH, N);
    default: return 0;
  }
}

// Per-block increments of the causal state for bf16 inputs (agg [BH][nblk][D][M],
// aggz [BH][nblk][D]; blocks of tblk tokens, tblk a multiple of 128).
hipError_t launch_block_state_bf16(const void* k, const void* v, int BH, int N, int D, int M, int tblk, int nblk,
                                   float* agg, float* aggz, hipStream_t stream) {
  const dim3 grid((unsigned)nblk * (unsigned)BH), block(nc::NT);
#define LA_NC_STATE(DD, MM)                                                                                  \
  hipLaunchKernelGGL((nc::nc_state_kernel<DD, MM>), grid, block, 0, stream, (const bf16_t*)k, (const bf16_t*)v, \
                     N, tblk, nblk, agg, aggz, DD * MM, DD)
  switch (D * 100 + M) {
    case 3232: LA_NC_STATE(32, 32); break;
    case 3264: LA_NC_STATE(32, 64); break;
    case 6432: LA_NC_STATE(64, 32); break;
    case 6464: LA_NC_STATE(64, 64); break;
    default: return hipErrorInvalidValue;
  }
#undef LA_NC_STATE
  return hipGetLastError();
}

hipError_t launch_noncausal_bf16(const void* q, const void* k, const void* v, void* o, int BH, int N, int D, int M,
                                 void* ws, hipStream_t stream) {
  switch (D * 100 + M) {
    case 3232: return nc::impl<32, 32>(q, k, v, o, BH, N, ws, stream);
    case 3264: return nc::impl<32, 64>(q, k, v, o, BH, N, ws, stream);
    case 6432: return nc::impl<64, 32>(q, k, v, o, BH, N, ws, stream);
    case 6464: return nc::impl<64, 64>(q, k, v, o, BH, N, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
