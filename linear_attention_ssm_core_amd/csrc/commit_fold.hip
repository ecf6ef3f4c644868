// Commit of a verify's accepted prefix, and the fold of a write-on-accept
// verify's accepted rows (gdn_fold_accepted on the
// metrale_model_layers/layers/qwen3_ssm/trait_layer.rs page; gdn_wy4_fold_k on the
// layer_struct.rs page).  Both also advance the conv state over the accepted rows.
#include "recurrent_kernel.h"

namespace gdn {
namespace {

// The state copy of a sequence is split into tiles of 256 16-byte vectors (4 KiB),
// one vector per thread: many short workgroups, dispatched in address order, keep
// the copies that are in flight at any moment close together, an order the HBM
// read and write streams serve faster than long workgroups each sweeping its own
// region (a cache-cold 4 GiB copy: 6.2 TB/s with one vector per thread, 5.3 with
// sixteen).  blockIdx.x < the tile count copies a tile; the rest rebuild
// conv-state channels; blockIdx.y is the sequence.
constexpr int kCommitTile = 256;  // 16-byte vectors per copy workgroup
constexpr int kMaxFoldRows = 16;

// The conv state of sequence i becomes the last K-1 rows of
// [old conv state ; its first na rows]; channel c = cblk * 256 + threadIdx.x.
template <typename TE>
__device__ __forceinline__ void advance_ring(const Geometry &geo, void *const *conv_state, const void *xv,
                                             const int32_t *cu, int i, int na, int cblk) {
  const int C = geo.conv_dim, R = geo.K - 1;
  const int c = cblk * 256 + threadIdx.x;
  if (c >= C) return;
  TE *ring = static_cast<TE *>(conv_state[i]);
  const TE *x = static_cast<const TE *>(xv) + (size_t)cu[i] * C;
  TE vals[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) {  // position na + r of [old conv state ; accepted rows]
    const int idx = na + min(r, R - 1);
    const TE vr = ring[(size_t)min(idx, R - 1) * C + c], vx = x[(size_t)max(idx - R, 0) * C + c];
    vals[r] = (idx < R) ? vr : vx;
  }
#pragma unroll
  for (int r = 0; r < 3; ++r)
    if (r < R) ring[(size_t)r * C + c] = vals[r];
}

// Commit: copy the state after the last accepted row into table 0.
template <typename TE>
__global__ __launch_bounds__(256) void commit_kernel(CommitLaunch p, int64_t n4, int ntiles) {
  const int i = blockIdx.y;
  const int k = p.cu[i + 1] - p.cu[i];
  const int na = p.n_accepted[i];
  if (na < 1 || na > k) return;  // outside the caller's contract: sequence untouched
  if ((int)blockIdx.x < ntiles) {
    if (na == k) return;  // table 0 already holds the last state
    // (native 4-float vectors: the struct-based float4 array ends up in scratch)
    const gptr<const floatx4> src = to_global(static_cast<const floatx4 *>(p.tables[na * kTableSeqs + i]));
    const gptr<floatx4> dst = to_global(static_cast<floatx4 *>(p.tables[i]));
    const int64_t idx = (int64_t)blockIdx.x * kCommitTile + threadIdx.x;
    // non-temporal, as the other state streams (64 accepted states: 48.5 -> 42.5 us by events)
    if (idx < n4) __builtin_nontemporal_store(__builtin_nontemporal_load(&src[idx]), &dst[idx]);
  } else {
    advance_ring<TE>(p.geo, p.conv_state, p.x, p.cu, i, na, (int)blockIdx.x - ntiles);
  }
}

// Fold: blockIdx.y < H_v is one value head's state, advanced over the accepted
// rows from the stash in order (the verify's rank-1 update, in the same operation
// order) and written back; the other blocks advance the conv state.  Thread t owns
// column quad t % (D/4) of the rows state_row(t / (D/4), .), as in the verify.
// Every state element folds on its own (S_ij <- a_r S_ij + u_r[j] k_r[i], r in
// order), so a thread streams its rows through in slices of SL, the next slice's
// loads in flight while the current one is folded: 56 VGPRs (fp32 states, d = 128)
// instead of 113 with all RPT rows held, eight workgroups per CU instead of four,
// and the 2,048 workgroups of 64 sequences x 32 heads resident at once (53 against
// 55 us on one MI355X; slices of 4 rows: 54 us, of 8: 68 us with spills).
template <int D, typename TE, typename TS>
__global__ __launch_bounds__(kSlot) __attribute__((amdgpu_waves_per_eu(8))) void fold_kernel(FoldLaunch p) {
  constexpr int CQ = HeadLayout<D>::CQ, RPT = HeadLayout<D>::RPT;
  constexpr int SL = RPT < 2 ? RPT : 2, NSL = RPT / SL;  // rows per slice, slices
  __shared__ float s_k[kMaxFoldRows][D], s_u[kMaxFoldRows][D], s_a[kMaxFoldRows];
  const int i = blockIdx.x;
  const int r0 = p.cu[i];
  const int k = p.cu[i + 1] - r0;
  const int na = p.n_accepted[i];
  if (na < 1 || na > k || na > kMaxFoldRows) return;  // outside the caller's contract
  const int Hv = p.geo.Hv, Hk = p.geo.Hk;
  if ((int)blockIdx.y >= Hv) {
    advance_ring<TE>(p.geo, p.conv_state, p.x, p.cu, i, na, (int)blockIdx.y - Hv);
    return;
  }
  const int h = blockIdx.y, g = h / (Hv / Hk);
  const int t = threadIdx.x, cq = t % CQ, rg = t / CQ;
  const gptr<TS> S = to_global(static_cast<TS *>(p.states[i])) + (size_t)h * D * D + 4 * cq;
  typename StateIO<TS>::raw cur[SL], nxt[SL];
#pragma unroll
  for (int rr = 0; rr < SL; ++rr) cur[rr] = StateIO<TS>::load(S + (size_t)state_row<D>(rg, rr) * D);
  const gptr<const float> stash = to_global(p.stash) + (size_t)r0 * p.stash_row;
  for (int e = t; e < na * D; e += kSlot) {
    const int r = e / D, j = e - r * D;
    s_k[r][j] = stash[(size_t)r * p.stash_row + g * D + j];
    s_u[r][j] = stash[(size_t)r * p.stash_row + Hk * D + h * D + j];
  }
  if (t < na) s_a[t] = stash[(size_t)t * p.stash_row + Hk * D + Hv * D + h];
  __syncthreads();
#pragma unroll
  for (int sl = 0; sl < NSL; ++sl) {
    if (sl + 1 < NSL) {
#pragma unroll
      for (int rr = 0; rr < SL; ++rr) nxt[rr] = StateIO<TS>::load(S + (size_t)state_row<D>(rg, SL * (sl + 1) + rr) * D);
    }
    floatx4 v[SL];
#pragma unroll
    for (int rr = 0; rr < SL; ++rr) v[rr] = StateIO<TS>::widen(cur[rr]);
    for (int r = 0; r < na; ++r) {
      const float av = s_a[r];
      const floatx4 u = *reinterpret_cast<const floatx4 *>(&s_u[r][4 * cq]);
#pragma unroll
      for (int rr = 0; rr < SL; ++rr)
        v[rr] = StateIO<TS>::as_stored(rank1_update(v[rr], av, s_k[r][state_row<D>(rg, SL * sl + rr)], u));
    }
#pragma unroll
    for (int rr = 0; rr < SL; ++rr) StateIO<TS>::store(S + (size_t)state_row<D>(rg, SL * sl + rr) * D, v[rr]);
#pragma unroll
    for (int rr = 0; rr < SL; ++rr) cur[rr] = nxt[rr];
  }
}

template <int D, typename TE>
hipError_t launch_fold_ts(const FoldLaunch &p, hipStream_t stream) {
  const int nblk_ring = (p.geo.conv_dim + 255) / 256;
  const dim3 grid(p.n, p.geo.Hv + nblk_ring), block(kSlot);
  if (p.state_f16)
    hipLaunchKernelGGL((fold_kernel<D, TE, _Float16>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((fold_kernel<D, TE, float>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fold_d(const FoldLaunch &p, hipStream_t stream) {
  return p.geo.act_bf16 ? launch_fold_ts<D, uint16_t>(p, stream) : launch_fold_ts<D, float>(p, stream);
}

}  // namespace

hipError_t launch_commit(const CommitLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  // 16-byte vectors per sequence state: 4 fp32 or 8 binary16 elements each
  const int64_t n4 = (int64_t)p.geo.Hv * p.geo.D * p.geo.D / (p.state_f16 ? 8 : 4);
  const int ntiles = (int)((n4 + kCommitTile - 1) / kCommitTile);
  const int nblk_ring = (p.geo.conv_dim + 255) / 256;
  const dim3 grid(ntiles + nblk_ring, p.n), block(256);
  if (p.geo.act_bf16)
    hipLaunchKernelGGL((commit_kernel<uint16_t>), grid, block, 0, stream, p, n4, ntiles);
  else
    hipLaunchKernelGGL((commit_kernel<float>), grid, block, 0, stream, p, n4, ntiles);
  return hipGetLastError();
}

hipError_t launch_fold(const FoldLaunch &p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  switch (p.geo.D) {
    case 32: return launch_fold_d<32>(p, stream);
    case 64: return launch_fold_d<64>(p, stream);
    case 128: return launch_fold_d<128>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
