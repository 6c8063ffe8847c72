// Expert-parallel token exchange around the grouped FFN, the part one GPU
// can run: the send plan of a source rank, the receive plan and the regroup
// of received rows into local-expert-contiguous order (and back), and a
// loopback stand-in for the exchanges between ranks.
//
// The pages ask for expert parallelism combined with data parallelism where
// ranks hold different token counts or none at all, with the expert
// communication, its ordering and its buffer capacities handled inside the
// runtime (Support combined expert and data parallelism in TrainerRank,
// Desired behavior), and for an EP=2 run on unequal batches with an
// empty-work case (same page, Acceptance).
//
// Global expert g = r * E_local + e is local expert e of rank r. A source
// rank routes over all experts, so its dispatched rows are already one
// contiguous segment per destination; its send plan is its counts table
// [EP, E_local] and the segment starts. A destination numbers the rows it
// receives source-major and regroups them by local expert, then source, then
// their order in the segment. All counts stay on the device: the kernels
// take capacities from the host and row totals from device tables.
#include "common.h"
#include "kernels.h"

namespace moe {

// send_counts[i] = counts[i] (i < EP*E_local); send_offsets[r] =
// offsets[r*E_local], send_offsets[EP] = offsets[E]; zeros for an empty
// source (counts and offsets are then not read).
__global__ __launch_bounds__(256) void ep_send_plan_kernel(const int32_t *__restrict__ counts,
                                                           const int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ send_counts,
                                                           int32_t *__restrict__ send_offsets, int ep, int e_local,
                                                           int empty) {
  const int E = ep * e_local;
  for (int i = threadIdx.x; i < E; i += 256) send_counts[i] = empty ? 0 : counts[i];
  for (int r = threadIdx.x; r <= ep; r += 256) send_offsets[r] = empty ? 0 : offsets[r * e_local];
}

// Per destination, from recv_counts [EP, E_local]: local_counts[e] (sum over
// sources), local_offsets (exclusive scan, E_local+1 entries) and
// recv_offsets (rows of the sources before s, EP+1 entries). One workgroup;
// sums in a fixed order.
__global__ __launch_bounds__(256) void ep_recv_plan_kernel(const int32_t *__restrict__ rc,
                                                           int32_t *__restrict__ local_counts,
                                                           int32_t *__restrict__ local_offsets,
                                                           int32_t *__restrict__ recv_offsets, int ep, int e_local) {
  __shared__ int s_cnt[256];
  __shared__ int s_src[kEpMaxRanks];
  const int e = threadIdx.x;
  int c = 0;
  if (e < e_local)
    for (int s = 0; s < ep; ++s) c += rc[s * e_local + e];
  s_cnt[e] = c;
  if (e < ep) {
    int t = 0;
    for (int q = 0; q < e_local; ++q) t += rc[e * e_local + q];
    s_src[e] = t;
  }
  __syncthreads();
  if (e < e_local) local_counts[e] = c;
  if (e == 0) {
    int acc = 0;
    for (int q = 0; q < e_local; ++q) {
      local_offsets[q] = acc;
      acc += s_cnt[q];
    }
    local_offsets[e_local] = acc;
    acc = 0;
    for (int s = 0; s < ep; ++s) {
      recv_offsets[s] = acc;
      acc += s_src[s];
    }
    recv_offsets[ep] = acc;
  }
}

// regroup_row for the run of source s and local expert e (one workgroup per
// run): its received rows start at (rows of sources before s) + (rows of s
// for experts before e), its grouped rows at (rows of experts before e) +
// (rows of e from sources before s). Rows past the capacity are skipped
// rather than written, so a corrupted table cannot write out of bounds.
__global__ __launch_bounds__(256) void ep_regroup_map_kernel(const int32_t *__restrict__ rc,
                                                             int32_t *__restrict__ regroup_row, int64_t rows_cap,
                                                             int ep, int e_local) {
  __shared__ int s_red[2][256];
  const int run = blockIdx.x;
  const int s = run / e_local, e = run - s * e_local;
  const int n = rc[s * e_local + e];
  if (n <= 0) return;  // uniform across the workgroup
  int src0 = 0, dst0 = 0;
  for (int i = threadIdx.x; i < ep * e_local; i += 256) {
    const int si = i / e_local, ei = i - si * e_local;
    const int v = rc[i];
    if (si < s || (si == s && ei < e)) src0 += v;  // source-major order before this run
    if (ei < e || (ei == e && si < s)) dst0 += v;  // expert-major order before this run
  }
  s_red[0][threadIdx.x] = src0;
  s_red[1][threadIdx.x] = dst0;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      s_red[0][threadIdx.x] += s_red[0][threadIdx.x + o];
      s_red[1][threadIdx.x] += s_red[1][threadIdx.x + o];
    }
    __syncthreads();
  }
  const int64_t a = s_red[0][0], b = s_red[1][0];
  for (int j = threadIdx.x; j < n; j += 256)
    if (a + j < rows_cap && b + j < rows_cap) regroup_row[a + j] = (int32_t)(b + j);
}

// Row regroup of the received rows i < recv_offsets[EP]:
//   forward: dst[regroup_row[i]] = src[i];   reverse: dst[i] = src[regroup_row[i]].
// A workgroup takes whole rows (its row index math is uniform), its threads
// consecutive 16-byte chunks; the workgroups stride over the rows up to the
// device total, so a launch sized for the capacity costs nothing past it.
template <typename T>
__global__ __launch_bounds__(256) void ep_regroup_kernel(const T *__restrict__ src, T *__restrict__ dst,
                                                         const int32_t *__restrict__ map,
                                                         const int32_t *__restrict__ total, int64_t rows_cap, int nc,
                                                         int reverse) {
  constexpr int V = Elem<T>::kVec;
  const int64_t n = min((int64_t)*total, rows_cap);
  const int64_t ld = (int64_t)nc * V;
  for (int64_t i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t j = map[i];
    if ((uint64_t)j >= (uint64_t)rows_cap) continue;
    const T *from = src + (reverse ? j : i) * ld;
    T *to = dst + (reverse ? i : j) * ld;
    for (int c = threadIdx.x; c < nc; c += 256) st16(to + (int64_t)c * V, ld16(from + (int64_t)c * V));
  }
}

// Counts exchange stand-in: recv_counts[r][s*E_local + e] = send_counts[s][r*E_local + e].
__global__ __launch_bounds__(256) void ep_exchange_counts_kernel(EpPtrs send_counts, EpPtrs recv_counts, int ep,
                                                                 int e_local) {
  const int n = ep * ep * e_local;
  for (int i = threadIdx.x; i < n; i += 256) {
    const int r = i / (ep * e_local), rem = i - r * ep * e_local;
    const int s = rem / e_local, e = rem - s * e_local;
    static_cast<int32_t *>(recv_counts.p[r])[s * e_local + e] =
        static_cast<const int32_t *>(send_counts.p[s])[r * e_local + e];
  }
}

// Rows exchange stand-in for source s: its row i < send_offsets[EP] belongs
// to the destination r whose segment holds it; it is received as row
// recv_offsets_r[s] + (i - send_offsets[r]) of r, and lands at that row of
// r's buffer, or, when r's regroup map is given, straight at its grouped row
// regroup_row_r[received row] (one copy instead of an exchange plus a
// regroup; a multi-GPU peer write can do the same). reverse copies the same
// rows back. Grid-stride over the source's rows: the host sizes the launch
// from the source's row count; a workgroup takes one row (uniform index
// math), its threads consecutive 16-byte chunks.
template <typename T>
__global__ __launch_bounds__(256) void ep_exchange_rows_kernel(T *__restrict__ src, const int32_t *__restrict__ send_off,
                                                               int64_t src_cap, EpPtrs dst, EpPtrs recv_off,
                                                               EpPtrs regroup, EpCaps dst_cap, int s, int ep, int nc,
                                                               int reverse) {
  constexpr int V = Elem<T>::kVec;
  const int64_t i = blockIdx.x;
  if (i >= src_cap || i >= send_off[ep]) return;
  int r = 0;
  while (r + 1 < ep && i >= send_off[r + 1]) ++r;
  int64_t row = static_cast<const int32_t *>(recv_off.p[r])[s] + (i - send_off[r]);
  if ((uint64_t)row >= (uint64_t)dst_cap.n[r]) return;
  if (regroup.p[r]) {
    row = static_cast<const int32_t *>(regroup.p[r])[row];
    if ((uint64_t)row >= (uint64_t)dst_cap.n[r]) return;
  }
  const int64_t ld = (int64_t)nc * V;
  T *d = static_cast<T *>(dst.p[r]) + row * ld;
  T *o = src + i * ld;
  for (int c = threadIdx.x; c < nc; c += 256) {
    if (reverse)
      st16(o + (int64_t)c * V, ld16(d + (int64_t)c * V));
    else
      st16(d + (int64_t)c * V, ld16(o + (int64_t)c * V));
  }
}

// Workgroups of a row-strided copy over up to `rows` rows: at most 16 per
// CU, fewer for small capacities.
static unsigned stride_grid(int64_t rows) {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess && hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                                                hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  const int64_t want = rows;
  const int64_t cap = (int64_t)cus * 16;
  return (unsigned)(want < cap ? (want > 0 ? want : 1) : cap);
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_ep_send_plan(const int32_t *counts, const int32_t *offsets, int32_t *send_counts,
                               int32_t *send_offsets, int ep, int e_local, bool empty, hipStream_t s) {
  LaunchScope scope("ep_send_plan", s);
  ep_send_plan_kernel<<<1, 256, 0, s>>>(counts, offsets, send_counts, send_offsets, ep, e_local, empty ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_ep_recv_plan(const int32_t *recv_counts, int32_t *local_counts, int32_t *local_offsets,
                               int32_t *recv_offsets, int32_t *regroup_row, int64_t rows_cap, int ep, int e_local,
                               hipStream_t s) {
  {
    LaunchScope scope("ep_recv_plan", s);
    ep_recv_plan_kernel<<<1, 256, 0, s>>>(recv_counts, local_counts, local_offsets, recv_offsets, ep, e_local);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || rows_cap == 0) return err;
  {
    LaunchScope scope("ep_regroup_map", s);
    ep_regroup_map_kernel<<<dim3((unsigned)(ep * e_local)), 256, 0, s>>>(recv_counts, regroup_row, rows_cap, ep,
                                                                         e_local);
  }
  return hipGetLastError();
}

hipError_t launch_ep_regroup(const void *src, void *dst, const int32_t *regroup_row, const int32_t *total,
                             int64_t rows_cap, int d, bool bf16, bool reverse, hipStream_t s) {
  LaunchScope scope(reverse ? "ep_ungroup" : "ep_regroup", s);
  const int nc = d / (bf16 ? 8 : 4);
  const unsigned grid = stride_grid(rows_cap);
  if (bf16)
    ep_regroup_kernel<bf16_t><<<grid, 256, 0, s>>>((const bf16_t *)src, (bf16_t *)dst, regroup_row, total, rows_cap,
                                                   nc, reverse ? 1 : 0);
  else
    ep_regroup_kernel<float><<<grid, 256, 0, s>>>((const float *)src, (float *)dst, regroup_row, total, rows_cap, nc,
                                                  reverse ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_ep_exchange_counts(const EpPtrs &send_counts, const EpPtrs &recv_counts, int ep, int e_local,
                                     hipStream_t s) {
  LaunchScope scope("ep_exchange_counts", s);
  ep_exchange_counts_kernel<<<1, 256, 0, s>>>(send_counts, recv_counts, ep, e_local);
  return hipGetLastError();
}

hipError_t launch_ep_exchange_rows(void *src, const int32_t *send_off, int64_t src_cap, const EpPtrs &dst,
                                   const EpPtrs &recv_off, const EpPtrs &regroup, const EpCaps &dst_cap, int source,
                                   int ep, int d, bool bf16, bool reverse, hipStream_t s) {
  if (src_cap == 0) return hipSuccess;
  LaunchScope scope(reverse ? "ep_return_rows" : "ep_exchange_rows", s);
  const int nc = d / (bf16 ? 8 : 4);
  const unsigned grid = (unsigned)src_cap;  // one workgroup per row the source can hold (< 2^24)
  if (bf16)
    ep_exchange_rows_kernel<bf16_t><<<grid, 256, 0, s>>>((bf16_t *)src, send_off, src_cap, dst, recv_off, regroup,
                                                         dst_cap, source, ep, nc, reverse ? 1 : 0);
  else
    ep_exchange_rows_kernel<float><<<grid, 256, 0, s>>>((float *)src, send_off, src_cap, dst, recv_off, regroup,
                                                        dst_cap, source, ep, nc, reverse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
