// Softmax over sink tokens and a sliding window at every position of a
// sequence (the prefill form of the exact path), gfx950.
// "The Key to Going Linear: Analysis-Driven Transformer Linearization",
// section 4 ("Adding Sliding Window Attention"): position t attends to the
// first s tokens and the w most recent ones (t itself included),
//   I_t = {0 .. s-1} u {t-w+1 .. t}   (0-based, each position once),
//   y_t = sum_{i in I_t} exp(sm q_t.k_i) v_i / sum_{i in I_t} exp(sm q_t.k_i),
// with the section 3.1 softmax restricted to I_t.  The layer output adds the
// linear path's read-out of the tokens in neither set.
//
// Dense contraction on MFMA.  One work-group of 8 waves per (b, h) and 128
// consecutive queries; wave w owns queries t0 + 16 w .. + 15.  Keys come in
// blocks of 64, staged in LDS (K as bf16, V converted to f16, exact for
// unit-scale values), the next block's global loads in flight while the
// current one is used.  Per block and wave:
//   S^T = K Q^T      bf16 MFMA 16x16x32; lane 16 g + r holds keys
//                    16 tt + 4 g + i of query r, so each lane owns one query
//   online softmax   base-2 exponent, running reference / partial sum per
//                    lane, merged over the 4 lane groups of a query by
//                    shuffles; the reference is raised (and O rescaled) only
//                    when a block's max exceeds it by more than 2^8
//   O^T += V^T P^T   f16 MFMA; P^T is the S^T accumulator pair of a 32-key
//                    step as is (keys 4 g + i and 16 + 4 g + i in lane group
//                    g), and the V^T operand gathers the same keys of one
//                    value column with LDS transpose reads
// A wave skips a block that holds none of its queries' keys and masks only
// blocks that are partly outside the set.  Work-groups of one (b, h) are
// placed on one XCD so their overlapping key blocks share its L2.
#include "gdn_f16ops.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

using namespace f16ops;

constexpr int PQ = 128;   // queries per work-group
constexpr int PK = 64;    // keys per block
constexpr int PD = 128;   // head dim
constexpr int PRS = 144;  // 16-bit row stride of the LDS tiles (288 bytes)
constexpr int PNT = 512;  // threads per work-group
constexpr float kLazy = 8.f;  // base-2 headroom before the softmax reference is raised

struct __align__(16) SwaPSmem {
  bf16 K[2][PK * PRS];
  h16 V[2][PK * PRS];
};

template <int X>
__device__ __forceinline__ float xor_lanes(float v) {
  return __shfl_xor(v, X);
}

template <class TOut>
__device__ __forceinline__ void store_row4(TOut* p, f32x4 o, bool add) {
  if constexpr (sizeof(TOut) == 2) {
    bf16x4* d = reinterpret_cast<bf16x4*>(p);
    if (add) {
      const bf16x4 c = *d;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] += (float)c[i];
    }
    bf16x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = (bf16)o[i];
    *d = v;
  } else {
    f32x4* d = reinterpret_cast<f32x4*>(p);
    if (add) o += *d;
    *d = o;
  }
}

// Rows t >= acc_from add y to out (out += y); rows below it are written.
template <class TOut>
__global__ __launch_bounds__(PNT, 2) void swa_sink_prefill_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    TOut* __restrict__ out, int T, int H, int n_sink, int window, float sm_log2,
    int acc_from, int nqb) {
  __shared__ SwaPSmem sm;
  int bh, qb;
  xcd_group_map(blockIdx.x, gridDim.x / nqb, nqb, &bh, &qb);
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, r = l & 15, g = l >> 4;
  const int t0 = qb * PQ;
  const int tq0 = t0 + 16 * w;  // first query of this wave
  const size_t rs = (size_t)H * PD;  // elements between consecutive tokens
  const size_t base = ((size_t)b * T * H + h) * PD;

  // Key blocks: the sink blocks below the first window block, then every
  // block from the earliest window start to the last query.  The window
  // blocks are visited in the order of their index modulo npd, the most
  // window blocks a work-group can have: the work-groups of one (b, h) start
  // together and move one block per step, so at step j all of them read the
  // blocks congruent to j -- a block's five or so readers fetch it at about
  // the same time and its later reads hit in L2.  (In index order, each
  // work-group would read a different block at every step and the whole
  // sequence's K and V would be live in L2 at once.)  The softmax is the
  // same in any order.
  const int kb_lo = max(0, t0 - window + 1) / PK;
  const int kb_hi = (min(T, t0 + PQ) - 1) / PK;
  const int nsb = min((n_sink + PK - 1) / PK, kb_lo);
  const int nwin = kb_hi - kb_lo + 1;
  const int nblk = nsb + nwin;
  const int npd = PQ / PK + (window - 1 + PK - 1) / PK;
  int rot = (npd - kb_lo % npd) % npd;  // position of the first block congruent to 0
  if (rot >= nwin) rot = 0;
  auto blk = [&](int i) {
    if (i < nsb) return i;
    int j = i - nsb + rot;
    if (j >= nwin) j -= nwin;
    return kb_lo + j;
  };

  // Q^T operand of this wave (query r, dims 32 j + 8 g .. + 7).
  bf16x8 qf[4];
  {
    const int tq = min(tq0 + r, T - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qf[j] = *reinterpret_cast<const bf16x8*>(q + base + (size_t)tq * rs + 32 * j + 8 * g);
  }

  // Staging: thread tid moves 16-byte pieces c = tid + PNT u of the block
  // (row c / 16, columns 8 (c % 16) ..), rows past T repeat row T - 1.
  constexpr int NST = PK * PD / 8 / PNT;  // pieces per thread and tensor
  static_assert(NST * PNT * 8 == PK * PD, "the threads cover the block exactly");
  bf16x8 kst[NST], vst[NST];
  auto fetch = [&](int kb) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int c = tid + PNT * u;
      const int key = min(kb * PK + (c >> 4), T - 1);
      const size_t off = base + (size_t)key * rs + 8 * (c & 15);
      kst[u] = *reinterpret_cast<const bf16x8*>(k + off);
      vst[u] = *reinterpret_cast<const bf16x8*>(v + off);
    }
  };
  auto stage = [&](int slot) {
#pragma unroll
    for (int u = 0; u < NST; ++u) {
      const int c = tid + PNT * u;
      const int o = (c >> 4) * PRS + 8 * (c & 15);
      *reinterpret_cast<bf16x8*>(&sm.K[slot][o]) = kst[u];
      *reinterpret_cast<h16x8*>(&sm.V[slot][o]) = bf16x8_to_h8(vst[u]);
    }
  };

  f32x4 acc_o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) acc_o[dt] = zero4();
  float m_run = -INFINITY, l_part = 0.f;
  const int tq = tq0 + r;  // this lane's query

  fetch(blk(0));
  for (int i = 0; i < nblk; ++i) {
    const int slot = i & 1;
    stage(slot);
    if (i + 1 < nblk) fetch(blk(i + 1));
    lds_barrier();

    const int k0 = blk(i) * PK;
    const bool skip = (k0 > tq0 + 15) || (k0 >= n_sink && k0 + PK - 1 <= tq0 - window);
    if (skip) continue;
    const bool full = (k0 + PK - 1 <= tq0) && (k0 > tq0 + 15 - window || k0 + PK - 1 < n_sink);

    // S^T = K Q^T for the 64 keys of the block.
    f32x4 s[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = zero4();
      const bf16* kr = &sm.K[slot][(16 * tt + r) * PRS + 8 * g];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        s[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(kr + 32 * j),
                                                         qf[j], s[tt], 0, 0, 0);
    }
    // Block max of the raw scores (the scale is positive, so it commutes
    // with the max), then p = 2^(sm_log2 s - m) with one FMA per score.
    float mloc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (!full) {
          const int key = k0 + 16 * tt + 4 * g + ii;
          const bool ok = key <= tq && (key < n_sink || key > tq - window);
          s[tt][ii] = ok ? s[tt][ii] : -INFINITY;
        }
        mloc = fmaxf(mloc, s[tt][ii]);
      }
    mloc = fmaxf(mloc, xor_lanes<16>(mloc));
    mloc = fmaxf(mloc, xor_lanes<32>(mloc));
    const float mblk = mloc * sm_log2;
    // Lazy reference: the running reference m_run is raised only when a
    // block's max exceeds it by more than kLazy (so p <= 2^kLazy); numerator
    // and denominator share the reference, so the result is unchanged.
    if (__any(mblk > m_run + kLazy)) {
      const float m_new = fmaxf(m_run, mblk);
      const float corr = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
      m_run = m_new;
      l_part *= corr;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) acc_o[dt] *= corr;
    }
    const float m_neg = m_run == -INFINITY ? 0.f : -m_run;
    float psum = 0.f;
    h16x4 pf[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      f32x4 p;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        p[ii] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][ii], sm_log2, m_neg));
        psum += p[ii];
      }
      pf[tt] = cvt4(p);
    }
    l_part += psum;

    // O^T += V^T P^T over two 32-key steps.
    const h16* vb = &sm.V[slot][(4 * g + (r >> 2)) * PRS + 4 * (r & 3)];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      const h16x8 pb = cat8(pf[2 * sp], pf[2 * sp + 1]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const h16* p = vb + 32 * sp * PRS + 16 * dt;
        const h16x8 va = cat8(ld_tr(p), ld_tr(p + 16 * PRS));
        acc_o[dt] = mfma32(va, pb, acc_o[dt]);
      }
    }
  }

  // Normalise and store: lane 16 g + r holds columns 16 dt + 4 g .. + 3 of
  // query tq.
  float lt = l_part + xor_lanes<16>(l_part);
  lt += xor_lanes<32>(lt);
  if (tq < T) {
    const float inv = 1.f / lt;
    TOut* orow = out + base + (size_t)tq * rs + 4 * g;
    const bool add = tq >= acc_from;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) store_row4<TOut>(orow + 16 * dt, acc_o[dt] * inv, add);
  }
}

// Decode-cache fill from a sequence's keys and values: slot j < n_sink holds
// position j, the position p >= n_sink lives in slot n_sink + (p - n_sink) %
// window; after T tokens the cache holds the sinks and the last `window`
// non-sink positions.  kFillParts work-groups per (b, h), each taking every
// kFillParts-th 256-piece stretch of its rows (one work-group per (b, h)
// left half of the CUs idle at B4 H32); 16-byte pieces, D / 8 or D / 4 per
// row.
constexpr int kFillParts = 8;
template <class T_>
__global__ __launch_bounds__(256) void swa_cache_fill_kernel(
    const T_* __restrict__ k, const T_* __restrict__ v, T_* __restrict__ kc,
    T_* __restrict__ vc, int T, int H, int D, int n_sink, int window) {
  const int bh = blockIdx.x / kFillParts, part = blockIdx.x % kFillParts;
  const int b = bh / H, h = bh % H;
  const int ns = min(n_sink, T);
  const int p_lo = max(n_sink, T - window);
  const int nw = max(0, T - p_lo);
  const int rows = ns + nw;
  constexpr int E = 16 / sizeof(T_);  // elements per 16-byte piece
  const int ppr = D / E;              // pieces per row
  for (int c = part * blockDim.x + threadIdx.x; c < rows * ppr; c += kFillParts * blockDim.x) {
    const int row = c / ppr, e = (c % ppr) * E;
    const int p = row < ns ? row : p_lo + (row - ns);
    const int slot = p < n_sink ? p : n_sink + (p - n_sink) % window;
    const size_t src = (((size_t)b * T + p) * H + h) * D + e;
    const size_t dst = ((size_t)bh * (n_sink + window) + slot) * D + e;
    *reinterpret_cast<f32x4*>(kc + dst) = *reinterpret_cast<const f32x4*>(k + src);
    *reinterpret_cast<f32x4*>(vc + dst) = *reinterpret_cast<const f32x4*>(v + src);
  }
}

}  // namespace

hipError_t launch_swa_prefill(const SwaPrefillArgs& p) {
  if ((long long)p.B * p.H * p.T == 0) return hipSuccess;
  const int nqb = (p.T + PQ - 1) / PQ;
  const float sm_log2 = p.softmax_scale * 1.4426950408889634f;
  const dim3 grid(p.B * p.H * nqb), block(PNT);
  const hipStream_t st = (hipStream_t)p.stream;
  if (p.out_bf16)
    hipLaunchKernelGGL(swa_sink_prefill_kernel<bf16>, grid, block, 0, st, (const bf16*)p.q,
                       (const bf16*)p.k, (const bf16*)p.v, (bf16*)p.out, p.T, p.H, p.n_sink,
                       p.window, sm_log2, p.acc_from, nqb);
  else
    hipLaunchKernelGGL(swa_sink_prefill_kernel<float>, grid, block, 0, st, (const bf16*)p.q,
                       (const bf16*)p.k, (const bf16*)p.v, (float*)p.out, p.T, p.H, p.n_sink,
                       p.window, sm_log2, p.acc_from, nqb);
  return hipGetLastError();
}

hipError_t launch_swa_cache_fill(const SwaCacheFillArgs& p) {
  if ((long long)p.B * p.H * p.T == 0) return hipSuccess;
  const dim3 grid(p.B * p.H * kFillParts), block(256);
  const hipStream_t st = (hipStream_t)p.stream;
  if (p.bf16)
    hipLaunchKernelGGL(swa_cache_fill_kernel<bf16>, grid, block, 0, st, (const bf16*)p.k,
                       (const bf16*)p.v, (bf16*)p.k_cache, (bf16*)p.v_cache, p.T, p.H, p.D,
                       p.n_sink, p.window);
  else
    hipLaunchKernelGGL(swa_cache_fill_kernel<float>, grid, block, 0, st, (const float*)p.k,
                       (const float*)p.v, (float*)p.k_cache, (float*)p.v_cache, p.T, p.H, p.D,
                       p.n_sink, p.window);
  return hipGetLastError();
}

}  // namespace gdn
