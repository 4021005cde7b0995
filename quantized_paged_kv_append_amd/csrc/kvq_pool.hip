// kvq_pool.hip -- device-side block pool: fixed-size blocks handed to
// sequences on demand, with a per-sequence logical-to-physical block table
// and the slot of every new token ("KV Cache Optimization: Strategies for
// Faster LLM Inference", section "How vLLM Implements KV Cache Optimization";
// "Dynamic KV Cache Quantization for Fast LLM Inference", section
// "Integrating Dynamic Quantization with PagedAttention").
//
// The pool is a stack of free block ids. A reservation is one workgroup: an
// exclusive scan of the per-sequence block needs (in batch order) decides,
// all or nothing, which stack positions each sequence takes, so the result is
// a pure function of the inputs. Latency-bound (a few microseconds per step).
#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_sharing.h"

namespace kvq {
namespace {

constexpr int kThreads = 1024;

// Block-wide exclusive scan of one int64 per thread; returns the prefix and
// writes the total to *total (all threads). Each wave scans its 64 values
// with shuffles, the wave totals meet in sh[0 .. kThreads / 64), and the
// trailing barrier frees sh for the next call: two barriers per scan.
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* total, int64_t* sh) {
  constexpr int kWaves = kThreads / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int64_t x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int64_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) sh[wave] = x;
  __syncthreads();
  // lane w < kWaves holds wave w's total; sums over the first kWaves lanes
  const int64_t t = lane < kWaves ? sh[lane] : 0;
  int64_t before = lane < wave ? t : 0, all = t;
#pragma unroll
  for (int off = 1; off < kWaves; off <<= 1) {
    before += __shfl_xor(before, off);
    all += __shfl_xor(all, off);
  }
  *total = __shfl(all, 0);
  before = __shfl(before, 0);
  __syncthreads();
  return before + x - v;
}

// Largest i < cnt with pre[i] <= f, for a non-decreasing pre with pre[0] = 0
// <= f: the entry whose run [pre[i], pre[i + 1]) holds f.
__device__ __forceinline__ int find_run(const int64_t* pre, int cnt, int64_t f) {
  int lo = 0, hi = cnt - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= f)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) void pool_init_kernel(int32_t* stack, int32_t* top,
                                                             const int32_t* order, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    stack[i] = order ? order[i] : (int32_t)i;
  if (blockIdx.x == 0 && threadIdx.x == 0) *top = (int32_t)n;
}

__device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

// Sequences are processed in chunks of kThreads, carrying the running block
// and token offsets, so any batch size works in one workgroup.
__global__ __launch_bounds__(kThreads) void reserve_kernel(
    int32_t* stack, int32_t* top, int32_t* tables, int32_t max_blocks,
    const int32_t* lens, const int32_t* new_tokens, int32_t batch, int32_t bs,
    int64_t* slots, int32_t* lens_out, int32_t* status, int64_t capacity,
    int64_t slot_capacity) {
  __shared__ int64_t sh[kThreads];
  __shared__ int64_t s_bpre[kThreads], s_wpre[kThreads], s_tout[kThreads];
  __shared__ int32_t s_L[kThreads], s_n[kThreads];
  __shared__ int ok_sh;
  const int tid = threadIdx.x;
  // a top outside [0, capacity] (a broken precondition) is cut to it
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  // pass 1: total need, table capacity check, and the slots the call writes
  if (tid == 0) ok_sh = 1;
  __syncthreads();
  int64_t total_need = 0, total_tok = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    int64_t need = 0, n = 0;
    if (b < batch) {
      n = new_tokens[b];
      const int64_t have = ceil_div(lens[b], bs);
      const int64_t want = ceil_div((int64_t)lens[b] + n, bs);
      if (want > max_blocks) ok_sh = 0;
      need = want - have;
    }
    int64_t chunk_total, chunk_tok;
    block_exclusive_scan(need, &chunk_total, sh);
    block_exclusive_scan(n, &chunk_tok, sh);
    total_need += chunk_total;
    total_tok += chunk_tok;
  }
  __syncthreads();
  if (total_tok > slot_capacity) {   // slot_mapping_out is too short: a caller error
    if (tid == 0) *status = KVQ_ERR_INVALID_ARGUMENT;
    return;
  }
  if (!ok_sh || total_need > top0) {
    if (tid == 0) *status = KVQ_ERR_OUT_OF_BLOCKS;
    return;
  }
  // pass 2, chunk by chunk: every thread of the workgroup writes table
  // entries and slots of any sequence of the chunk (runs found by a binary
  // search over the chunk's prefix sums), so a long prompt is placed in
  // parallel rather than by its own thread
  int64_t boff = 0, toff = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int cnt = min(kThreads, batch - base);
    int64_t L = 0, n = 0, need = 0, touched = 0;
    if (b < batch) {
      L = lens[b];
      n = new_tokens[b];
      need = ceil_div(L + n, bs) - ceil_div(L, bs);
      touched = n > 0 ? (L + n - 1) / bs - L / bs + 1 : 0;   // blocks the new tokens fall in
    }
    int64_t ctot, ttot, wtot;
    const int64_t bpre = block_exclusive_scan(need, &ctot, sh);
    const int64_t tpre = block_exclusive_scan(n, &ttot, sh);
    const int64_t wpre = block_exclusive_scan(touched, &wtot, sh);
    s_bpre[tid] = bpre;
    s_wpre[tid] = wpre;
    s_tout[tid] = toff + tpre;
    s_L[tid] = (int32_t)L;
    s_n[tid] = (int32_t)n;
    __syncthreads();
    // lengths may alias lens_out: each thread has read its own already
    if (b < batch && lens_out) lens_out[b] = (int32_t)(L + n);
    // sequence i takes the popped entries take0 .. take0 + need - 1, with
    // take0 = top0 - (boff + bpre_i) - need_i, as table entries have .. have + need - 1
    auto seq = [&](int i, int64_t& Li, int64_t& ni, int64_t& hi, int64_t& take0) {
      Li = s_L[i];
      ni = s_n[i];
      hi = ceil_div(Li, bs);
      take0 = top0 - (boff + s_bpre[i]) - (ceil_div(Li + ni, bs) - hi);
    };
    for (int64_t f = tid; f < ctot; f += kThreads) {
      const int i = find_run(s_bpre, cnt, f);
      int64_t Li, ni, hi, take0;
      seq(i, Li, ni, hi, take0);
      const int64_t k = f - s_bpre[i];
      tables[(int64_t)(base + i) * max_blocks + hi + k] = stack[take0 + k];
    }
    // slots, one touched block per iteration: its id from the row's existing
    // entries or the popped ones (never the entries written just above),
    // then its run of consecutive slots
    for (int64_t f = tid; f < wtot; f += kThreads) {
      const int i = find_run(s_wpre, cnt, f);
      int64_t Li, ni, hi, take0;
      seq(i, Li, ni, hi, take0);
      const int64_t blk = Li / bs + (f - s_wpre[i]);
      const int64_t id =
          blk < hi ? tables[(int64_t)(base + i) * max_blocks + blk] : stack[take0 + (blk - hi)];
      const int64_t p0 = max(Li, blk * bs), p1 = min(Li + ni, (blk + 1) * bs);
      int64_t* out = slots + s_tout[i] - Li;
      for (int64_t pos = p0; pos < p1; ++pos) out[pos] = id * bs + (pos - blk * bs);
    }
    boff += ctot;
    toff += ttot;
    __syncthreads();   // the chunk's arrays are read before the next chunk writes them
  }
  if (tid == 0) {
    *top = (int32_t)(top0 - total_need);
    *status = KVQ_OK;
  }
}

__global__ __launch_bounds__(kThreads) void release_kernel(
    int32_t* stack, int32_t* top, int64_t capacity, const int32_t* tables,
    int32_t max_blocks, const int32_t* lens, const int32_t* mask, int32_t batch,
    int32_t bs, int32_t* lens_out, int32_t* status) {
  __shared__ int64_t sh[kThreads];
  __shared__ int64_t s_pre[kThreads];
  const int tid = threadIdx.x;
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  int64_t total = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int64_t nb = (b < batch && mask[b]) ? min(ceil_div(lens[b], bs), (int64_t)max_blocks) : 0;
    int64_t t;
    block_exclusive_scan(nb, &t, sh);
    total += t;
  }
  if (top0 + total > capacity) {
    if (tid == 0) *status = KVQ_ERR_OUT_OF_BLOCKS;
    return;
  }
  // the chunk's released entries are spread over the whole workgroup (entry
  // f of the chunk belongs to the sequence whose prefix run holds it)
  int64_t off = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int cnt = min(kThreads, batch - base);
    const bool rel = b < batch && mask[b];
    const int64_t nb = rel ? min(ceil_div(lens[b], bs), (int64_t)max_blocks) : 0;
    int64_t t;
    s_pre[tid] = block_exclusive_scan(nb, &t, sh);
    __syncthreads();
    for (int64_t f = tid; f < t; f += kThreads) {
      const int i = find_run(s_pre, cnt, f);
      stack[top0 + off + f] = tables[(int64_t)(base + i) * max_blocks + (f - s_pre[i])];
    }
    off += t;
    __syncthreads();
  }
  // lengths are cleared only after every row has read its own length
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    if (lens_out && b < batch && mask[b]) lens_out[b] = 0;
  }
  if (tid == 0) {
    *top = (int32_t)(top0 + total);
    *status = KVQ_OK;
  }
}

// ---- prefix sharing --------------------------------------------------------
// refcount[id] counts the table entries holding block id; a free block has 0.
// Fork: one workgroup per fork copies the source row's entries to the
// destination row and counts them (device-scope atomics, so forks sharing a
// source may run at once).
__global__ __launch_bounds__(256) void fork_kernel(int32_t* refcount, int64_t capacity,
                                                   int32_t* tables, int32_t max_blocks,
                                                   int32_t* lens, int32_t batch,
                                                   const int32_t* src, const int32_t* dst,
                                                   int32_t bs) {
  const int k = blockIdx.x;
  const int s = src[k], d = dst[k];
  if (s < 0 || s >= batch || d < 0 || d >= batch || s == d) return;
  const int32_t L = lens[s];
  const int64_t nb = min(ceil_div(max(L, 0), bs), (int64_t)max_blocks);
  for (int64_t i = threadIdx.x; i < nb; i += blockDim.x) {
    const int32_t id = tables[(int64_t)s * max_blocks + i];
    tables[(int64_t)d * max_blocks + i] = id;
    if (id >= 0 && id < capacity) atomicAdd(&refcount[id], 1);
  }
  if (threadIdx.x == 0) lens[d] = L;
}

// A count after other waves' atomics on it: an L2-coherent load (a plain load
// could hit a line this CU cached before the atomics).
__device__ __forceinline__ int32_t count_now(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Copy on write of a shared, partly filled last block: whether sequence b
// copies, read from the counts at the start of the call.
__device__ __forceinline__ int cow_needed(const int32_t* refcount, int64_t capacity,
                                          const int32_t* tables, int32_t max_blocks,
                                          int b, int32_t L, int32_t n, int32_t bs) {
  if (n <= 0 || L % bs == 0 || L / bs >= max_blocks) return 0;
  const int32_t id = tables[(int64_t)b * max_blocks + L / bs];
  return id >= 0 && id < capacity && refcount[id] > 1;
}

// Reservation with counts (one workgroup): the plain reservation's scans plus
// one extra block per copying sequence, taken first; new blocks get count 1;
// then the copied blocks lose a reference each and those that reach zero are
// pushed in the order of their last copy. The last-copy test uses the count
// itself as scratch: after the decrements, every copy c of a block left at
// zero lowers its count to -(c + 1) with atomicMin, so the copy that finds
// -(c + 1) there is the last one; the counts are then reset to zero.
__global__ __launch_bounds__(kThreads) void reserve_shared_kernel(
    int32_t* stack, int32_t* top, int64_t capacity, int32_t* refcount, int32_t* tables,
    int32_t max_blocks, const int32_t* lens, const int32_t* new_tokens, int32_t batch,
    int32_t bs, int64_t* slots, int32_t* lens_out, int32_t* cow_src, int32_t* cow_dst,
    int32_t* cow_count, int32_t* status, int64_t slot_capacity) {
  __shared__ int64_t sh[kThreads];
  __shared__ int64_t s_first[kThreads], s_gpre[kThreads], s_xpre[kThreads], s_tout[kThreads];
  __shared__ int32_t s_L[kThreads], s_n[kThreads], s_cow[kThreads];
  __shared__ int ok_sh;
  const int tid = threadIdx.x;
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  if (tid == 0) ok_sh = 1;
  __syncthreads();
  int64_t total_need = 0, total_tok = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    int64_t need = 0, n = 0;
    if (b < batch) {
      n = new_tokens[b];
      const int64_t have = ceil_div(lens[b], bs);
      const int64_t want = ceil_div((int64_t)lens[b] + n, bs);
      if (want > max_blocks) ok_sh = 0;
      need = want - have +
             cow_needed(refcount, capacity, tables, max_blocks, b, lens[b], new_tokens[b], bs);
    }
    int64_t chunk_total, chunk_tok;
    block_exclusive_scan(need, &chunk_total, sh);
    block_exclusive_scan(n, &chunk_tok, sh);
    total_need += chunk_total;
    total_tok += chunk_tok;
  }
  __syncthreads();
  if (total_tok > slot_capacity) {   // slot_mapping_out is too short: a caller error
    if (tid == 0) *status = KVQ_ERR_INVALID_ARGUMENT;
    return;
  }
  if (!ok_sh || total_need > top0) {
    if (tid == 0) *status = KVQ_ERR_OUT_OF_BLOCKS;
    return;
  }
  // the copy decisions are taken before any count changes (pass 2 only sets
  // the counts of blocks taken from the stack, which no table holds). Table
  // entries and slots are spread over the workgroup as in reserve_kernel.
  int64_t boff = 0, toff = 0, coff = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int cnt = min(kThreads, batch - base);
    int64_t grow = 0, n = 0, L = 0, touched = 0;
    int cow = 0;
    if (b < batch) {
      L = lens[b];
      n = new_tokens[b];
      grow = ceil_div(L + n, bs) - ceil_div(L, bs);
      cow = cow_needed(refcount, capacity, tables, max_blocks, b, (int32_t)L, (int32_t)n, bs);
      touched = n > 0 ? (L + n - 1) / bs - L / bs + 1 : 0;
    }
    const int64_t need = grow + cow;
    int64_t ctot, ttot, wtot, gtot, xtot;
    const int64_t bpre = block_exclusive_scan(need, &ctot, sh) + boff;
    const int64_t tpre = block_exclusive_scan(n, &ttot, sh) + toff;
    const int64_t cpre = block_exclusive_scan(cow, &wtot, sh) + coff;
    const int64_t gpre = block_exclusive_scan(grow, &gtot, sh);
    const int64_t xpre = block_exclusive_scan(touched, &xtot, sh);
    // sequence i of the chunk takes stack entries first .. first + need - 1:
    // the copy's fresh block (if any), then its grown blocks
    const int64_t first = top0 - bpre - need;
    s_first[tid] = first;
    s_gpre[tid] = gpre;
    s_xpre[tid] = xpre;
    s_tout[tid] = tpre;
    s_L[tid] = (int32_t)L;
    s_n[tid] = (int32_t)n;
    s_cow[tid] = cow;
    __syncthreads();   // every copy decision of this chunk is read before counts change
    if (b < batch) {
      int32_t* row = tables + (int64_t)b * max_blocks;
      if (cow) {
        const int32_t fresh = stack[first];
        cow_src[cpre] = row[L / bs];
        cow_dst[cpre] = fresh;
        row[L / bs] = fresh;
        if (fresh >= 0 && fresh < capacity) refcount[fresh] = 1;
      }
      if (lens_out) lens_out[b] = (int32_t)(L + n);
    }
    for (int64_t f = tid; f < gtot; f += kThreads) {
      const int i = find_run(s_gpre, cnt, f);
      const int64_t k = f - s_gpre[i];
      const int32_t id = stack[s_first[i] + s_cow[i] + k];
      tables[(int64_t)(base + i) * max_blocks + ceil_div(s_L[i], bs) + k] = id;
      if (id >= 0 && id < capacity) refcount[id] = 1;
    }
    // slots block by block; a block's id is the row's existing entry, the
    // copy's fresh block (the partial block of a copying row) or a grown
    // one, never a re-read of an entry written in this pass
    for (int64_t f = tid; f < xtot; f += kThreads) {
      const int i = find_run(s_xpre, cnt, f);
      const int64_t Li = s_L[i], ni = s_n[i], hi = ceil_div(Li, bs);
      const int64_t blk = Li / bs + (f - s_xpre[i]);
      int64_t id;
      if (s_cow[i] && blk == Li / bs)
        id = stack[s_first[i]];
      else if (blk < hi)
        id = tables[(int64_t)(base + i) * max_blocks + blk];
      else
        id = stack[s_first[i] + s_cow[i] + (blk - hi)];
      const int64_t p0 = max(Li, blk * bs), p1 = min(Li + ni, (blk + 1) * bs);
      int64_t* out = slots + s_tout[i] - Li;
      for (int64_t pos = p0; pos < p1; ++pos) out[pos] = id * bs + (pos - blk * bs);
    }
    boff += ctot;
    toff += ttot;
    coff += wtot;
    __syncthreads();
  }
  const int64_t ncow = coff;
  const int64_t top1 = top0 - total_need;
  // copied blocks lose a reference
  for (int64_t c = tid; c < ncow; c += kThreads) {
    const int32_t id = cow_src[c];
    if (id >= 0 && id < capacity) atomicSub(&refcount[id], 1);
  }
  __syncthreads();
  for (int64_t c = tid; c < ncow; c += kThreads) {
    const int32_t id = cow_src[c];
    if (id >= 0 && id < capacity && count_now(&refcount[id]) <= 0)
      atomicMin(&refcount[id], (int32_t)(-(c + 1)));
  }
  __syncthreads();
  int64_t poff = 0;
  for (int64_t base = 0; base < ncow; base += kThreads) {
    const int64_t c = base + tid;
    const int32_t id = c < ncow ? cow_src[c] : -1;
    const int last = id >= 0 && id < capacity && count_now(&refcount[id]) == (int32_t)(-(c + 1));
    int64_t ptot;
    const int64_t pre = block_exclusive_scan(last, &ptot, sh) + poff;
    if (last && top1 + pre < capacity) stack[top1 + pre] = id;
    poff += ptot;
    __syncthreads();   // every test of this chunk is done before any reset
    if (last) refcount[id] = 0;
  }
  if (tid == 0) {
    *top = (int32_t)min(top1 + poff, capacity);
    *cow_count = (int32_t)ncow;
    *status = KVQ_OK;
  }
}

// Release with counts (one workgroup): the masked rows' table entries, in
// (row, logical block) order, are enumerated chunk by chunk (a scan of the
// rows' block counts, then a binary search per entry); every entry drops a
// reference; a block left at zero is pushed in the order of its last entry
// (the same atomicMin marking as in reserve_shared_kernel).
__device__ __forceinline__ int find_row(const int64_t* incl, int n, int64_t e) {
  int lo = 0, hi = n - 1;   // first row whose inclusive prefix exceeds e
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (incl[mid] > e) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

template <int PHASE>
__device__ void release_entries(int32_t* stack, int64_t top0, int64_t capacity,
                                int32_t* refcount, const int32_t* tables, int32_t max_blocks,
                                const int32_t* lens, const int32_t* mask, int32_t batch,
                                int32_t bs, int64_t* sh, int64_t* sh2, int64_t* pushed) {
  const int tid = threadIdx.x;
  int64_t ebase = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int64_t nb = (b < batch && mask[b]) ? min(ceil_div(max(lens[b], 0), bs), (int64_t)max_blocks) : 0;
    int64_t total;
    const int64_t pre = block_exclusive_scan(nb, &total, sh2);
    sh[tid] = pre + nb;   // inclusive prefix of this chunk's rows
    __syncthreads();
    const int rows = min(kThreads, batch - base);
    for (int64_t e0 = 0; e0 < total; e0 += kThreads) {
      const int64_t e = e0 + tid;
      int32_t id = -1;
      if (e < total) {
        const int r = find_row(sh, rows, e);
        const int64_t i = e - (r ? sh[r - 1] : 0);
        id = tables[(int64_t)(base + r) * max_blocks + i];
        if (id < 0 || id >= capacity) id = -1;
      }
      const int64_t E = ebase + e;   // entry index over the whole call
      if (PHASE == 0) {
        if (id >= 0) atomicSub(&refcount[id], 1);
      } else if (PHASE == 1) {
        if (id >= 0 && count_now(&refcount[id]) <= 0) atomicMin(&refcount[id], (int32_t)(-(E + 1)));
      } else {
        const int last = id >= 0 && count_now(&refcount[id]) == (int32_t)(-(E + 1));
        int64_t ptot;
        const int64_t p = block_exclusive_scan(last, &ptot, sh2) + *pushed;
        if (last && top0 + p < capacity) stack[top0 + p] = id;
        __syncthreads();   // every test of this batch of entries is done
        if (last) refcount[id] = 0;
        *pushed += ptot;
      }
    }
    ebase += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void release_shared_kernel(
    int32_t* stack, int32_t* top, int64_t capacity, int32_t* refcount, const int32_t* tables,
    int32_t max_blocks, const int32_t* lens, const int32_t* mask, int32_t batch, int32_t bs,
    int32_t* lens_out, int32_t* status) {
  __shared__ int64_t sh[kThreads];
  __shared__ int64_t sh2[kThreads];
  const int tid = threadIdx.x;
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  int64_t pushed = 0;
  release_entries<0>(stack, top0, capacity, refcount, tables, max_blocks, lens, mask, batch, bs,
                     sh, sh2, &pushed);
  __syncthreads();
  release_entries<1>(stack, top0, capacity, refcount, tables, max_blocks, lens, mask, batch, bs,
                     sh, sh2, &pushed);
  __syncthreads();
  release_entries<2>(stack, top0, capacity, refcount, tables, max_blocks, lens, mask, batch, bs,
                     sh, sh2, &pushed);
  __syncthreads();
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    if (lens_out && b < batch && mask[b]) lens_out[b] = 0;
  }
  if (tid == 0) {
    *top = (int32_t)min(top0 + pushed, capacity);
    *status = top0 + pushed <= capacity ? KVQ_OK : KVQ_ERR_OUT_OF_BLOCKS;
  }
}

// Window trimming (one workgroup): sequence b's blocks i in
// [ceil(sink / bs), floor((L + 1 - window) / bs)) that are still in its table
// are pushed (batch order, logical order) and their entries cleared; all or
// nothing if the pushes would overflow the stack.
__device__ __forceinline__ void trim_range(int32_t L, int32_t window, int32_t sink, int32_t bs,
                                           int32_t max_blocks, int64_t& lo, int64_t& hi) {
  lo = ceil_div(max(sink, 0), bs);
  hi = (int64_t)L + 1 - window >= 0 ? ((int64_t)L + 1 - window) / bs : 0;
  hi = min(hi, (int64_t)max_blocks);
}

// Entries [lo, hi) of every row of a chunk are enumerated by the whole
// workgroup in (row, block) order: entry e of the chunk belongs to the row
// whose run in the chunk's prefix sums holds it. PUSH = false counts the live
// (non-negative) entries; PUSH = true moves them to the stack from `pos` on,
// in that order, and clears them.
template <bool PUSH>
__device__ int64_t trim_entries(int32_t* stack, int64_t pos, int32_t* tables, int32_t max_blocks,
                                const int32_t* lens, int32_t window, int32_t sink, int32_t batch,
                                int32_t bs, int64_t* sh, int64_t* s_pre, int64_t* s_lo) {
  const int tid = threadIdx.x;
  int64_t live = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const int cnt = min(kThreads, batch - base);
    int64_t lo = 0, hi = 0;
    if (b < batch && window > 0) trim_range(lens[b], window, sink, bs, max_blocks, lo, hi);
    int64_t etot;
    s_pre[tid] = block_exclusive_scan(max(hi - lo, (int64_t)0), &etot, sh);
    s_lo[tid] = lo;
    __syncthreads();
    for (int64_t e0 = 0; e0 < etot; e0 += kThreads) {
      const int64_t e = e0 + tid;
      int32_t* ent = nullptr;
      int32_t id = -1;
      if (e < etot) {
        const int r = find_run(s_pre, cnt, e);
        ent = &tables[(int64_t)(base + r) * max_blocks + s_lo[r] + (e - s_pre[r])];
        id = *ent;
      }
      int64_t ktot;
      const int64_t k = block_exclusive_scan(id >= 0 ? 1 : 0, &ktot, sh);
      if (PUSH && id >= 0) {
        stack[pos + live + k] = id;
        *ent = -1;
      }
      live += ktot;
    }
    __syncthreads();   // the chunk's arrays are read before the next chunk writes them
  }
  return live;
}

__global__ __launch_bounds__(kThreads) void trim_kernel(int32_t* stack, int32_t* top,
                                                        int64_t capacity, int32_t* tables,
                                                        int32_t max_blocks, const int32_t* lens,
                                                        int32_t window, int32_t sink,
                                                        int32_t batch, int32_t bs,
                                                        int32_t* status) {
  __shared__ int64_t sh[kThreads];
  __shared__ int64_t s_pre[kThreads], s_lo[kThreads];
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  const int64_t total = trim_entries<false>(stack, top0, tables, max_blocks, lens, window, sink,
                                            batch, bs, sh, s_pre, s_lo);
  if (top0 + total > capacity) {
    if (threadIdx.x == 0) *status = KVQ_ERR_OUT_OF_BLOCKS;
    return;
  }
  trim_entries<true>(stack, top0, tables, max_blocks, lens, window, sink, batch, bs, sh, s_pre,
                     s_lo);
  if (threadIdx.x == 0) {
    *top = (int32_t)(top0 + total);
    *status = KVQ_OK;
  }
}

// Pack / unpack of blocks for offload: workgroup (block k, plane), 16-byte
// vectors between the plane's slice of block ids[k] and its place in the
// pack (block k at k * pack_bytes, planes in order).
struct PackPlanes {
  uint8_t* base[6];
  int64_t per_block[6];   // 0: plane unused
  int64_t offset[6];      // the plane's offset inside a packed block
  int64_t pack_bytes;
};

template <bool PACK>
__global__ __launch_bounds__(256) void pack_kernel(PackPlanes pp, const int32_t* ids,
                                                   uint8_t* packed, int64_t num_blocks) {
  const int k = blockIdx.x, plane = blockIdx.y;
  const int64_t per = pp.per_block[plane];
  if (per == 0) return;
  const int32_t id = ids[k];
  if (id < 0 || id >= num_blocks) return;
  u32x4* cache = reinterpret_cast<u32x4*>(pp.base[plane] + id * per);
  u32x4* pk = reinterpret_cast<u32x4*>(packed + k * pp.pack_bytes + pp.offset[plane]);
  for (int64_t i = threadIdx.x; i < per / 16; i += blockDim.x) {
    if (PACK)
      pk[i] = cache[i];
    else
      cache[i] = pk[i];
  }
}

// Copy of one layer's planes for each (src, dst) block pair: workgroup
// (pair, plane), 16-byte vectors; pairs past *count are skipped.
struct CopyPlanes {
  uint8_t* base[6];
  int64_t per_block[6];   // bytes of each plane per block (0: plane unused)
};

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyPlanes cp, const int32_t* src,
                                                          const int32_t* dst,
                                                          const int32_t* count,
                                                          int64_t num_blocks) {
  const int k = blockIdx.x, plane = blockIdx.y;
  if (k >= *count || cp.per_block[plane] == 0) return;
  const int32_t s = src[k], d = dst[k];
  if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) return;
  const int64_t per = cp.per_block[plane];
  const u32x4* from = reinterpret_cast<const u32x4*>(cp.base[plane] + s * per);
  u32x4* to = reinterpret_cast<u32x4*>(cp.base[plane] + d * per);
  for (int64_t i = threadIdx.x; i < per / 16; i += blockDim.x) to[i] = from[i];
}

// Debug checks of the caller's tables and slots (one workgroup, so the
// smallest offending index comes from a block-wide minimum: no atomics, the
// same answer every run).
__device__ int64_t block_min_i64(int64_t v, int64_t* sh) {
  constexpr int kWaves = kThreads / kWave;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) v = min(v, (int64_t)__shfl_xor(v, off));
  if (lane == 0) sh[wave] = v;
  __syncthreads();
  int64_t m = lane < kWaves ? sh[lane] : INT64_MAX;
#pragma unroll
  for (int off = 1; off < kWaves; off <<= 1) m = min(m, (int64_t)__shfl_xor(m, off));
  return m;
}

__global__ __launch_bounds__(kThreads) void check_tables_kernel(
    const int32_t* tables, int32_t max_blocks, const int32_t* lens, int32_t batch, int32_t bs,
    int64_t num_blocks, int64_t* first_bad, int32_t* status) {
  __shared__ int64_t sh[kThreads / kWave];
  int64_t best = INT64_MAX;
  const int64_t total = (int64_t)batch * max_blocks;
  for (int64_t f = threadIdx.x; f < total; f += kThreads) {
    const int64_t b = f / max_blocks, k = f % max_blocks;
    const int64_t L = lens[b];
    bool bad;
    if (L < 0 || L > (int64_t)max_blocks * bs) {
      bad = k == 0;   // the length itself: reported at the row's first entry
    } else {
      const int32_t id = tables[f];
      bad = k < ceil_div(L, bs) && (id < 0 || id >= num_blocks);
    }
    if (bad) best = min(best, f);
  }
  best = block_min_i64(best, sh);
  if (threadIdx.x == 0) {
    *first_bad = best == INT64_MAX ? -1 : best;
    *status = best == INT64_MAX ? KVQ_OK : KVQ_ERR_INVALID_ARGUMENT;
  }
}

__global__ __launch_bounds__(kThreads) void check_slots_kernel(
    const int64_t* slots, int64_t n, int64_t limit, int64_t* first_bad, int32_t* status) {
  __shared__ int64_t sh[kThreads / kWave];
  int64_t best = INT64_MAX;
  for (int64_t t = threadIdx.x; t < n; t += kThreads) {
    const int64_t s = slots[t];
    if (s < -1 || s >= limit) best = min(best, t);
  }
  best = block_min_i64(best, sh);
  if (threadIdx.x == 0) {
    *first_bad = best == INT64_MAX ? -1 : best;
    *status = best == INT64_MAX ? KVQ_OK : KVQ_ERR_INVALID_ARGUMENT;
  }
}

}  // namespace

hipError_t launch_check_tables(const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                               int32_t batch, int32_t bs, int64_t num_blocks, int64_t* first_bad,
                               int32_t* status, hipStream_t stream) {
  check_tables_kernel<<<1, kThreads, 0, stream>>>(tables, max_blocks, lens, batch, bs,
                                                  num_blocks, first_bad, status);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t* slots, int64_t n, int64_t num_blocks, int32_t bs,
                              int64_t* first_bad, int32_t* status, hipStream_t stream) {
  check_slots_kernel<<<1, kThreads, 0, stream>>>(slots, n, num_blocks * bs, first_bad, status);
  return hipGetLastError();
}

hipError_t launch_pool_init(int32_t* stack, int32_t* top, const int32_t* order,
                            int64_t n, hipStream_t stream) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  pool_init_kernel<<<(int)blocks, kThreads, 0, stream>>>(stack, top, order, n);
  return hipGetLastError();
}

hipError_t launch_blocks_reserve(int32_t* stack, int32_t* top, int64_t capacity,
                                 int32_t* tables, int32_t max_blocks,
                                 const int32_t* lens, const int32_t* new_tokens,
                                 int32_t batch, int32_t bs, int64_t* slots,
                                 int64_t slot_capacity, int32_t* lens_out, int32_t* status,
                                 hipStream_t stream) {
  reserve_kernel<<<1, kThreads, 0, stream>>>(stack, top, tables, max_blocks, lens,
                                             new_tokens, batch, bs, slots, lens_out,
                                             status, capacity, slot_capacity);
  return hipGetLastError();
}

hipError_t launch_blocks_release(int32_t* stack, int32_t* top,
                                 int64_t capacity, const int32_t* tables,
                                 int32_t max_blocks, const int32_t* lens,
                                 const int32_t* mask, int32_t batch, int32_t bs,
                                 int32_t* lens_out, int32_t* status,
                                 hipStream_t stream) {
  release_kernel<<<1, kThreads, 0, stream>>>(stack, top, capacity, tables, max_blocks,
                                             lens, mask, batch, bs, lens_out, status);
  return hipGetLastError();
}

hipError_t launch_blocks_trim(int32_t* stack, int32_t* top, int64_t capacity, int32_t* tables,
                              int32_t max_blocks, const int32_t* lens, int32_t window,
                              int32_t sink, int32_t batch, int32_t bs, int32_t* status,
                              hipStream_t stream) {
  trim_kernel<<<1, kThreads, 0, stream>>>(stack, top, capacity, tables, max_blocks, lens, window,
                                          sink, batch, bs, status);
  return hipGetLastError();
}

hipError_t launch_blocks_fork(int32_t* refcount, int64_t capacity, int32_t* tables,
                              int32_t max_blocks, int32_t* lens, int32_t batch,
                              const int32_t* src, const int32_t* dst, int32_t num_forks,
                              int32_t bs, hipStream_t stream) {
  fork_kernel<<<num_forks, 256, 0, stream>>>(refcount, capacity, tables, max_blocks, lens,
                                             batch, src, dst, bs);
  return hipGetLastError();
}

hipError_t launch_blocks_reserve_shared(int32_t* stack, int32_t* top, int64_t capacity,
                                        int32_t* refcount, int32_t* tables, int32_t max_blocks,
                                        const int32_t* lens, const int32_t* new_tokens,
                                        int32_t batch, int32_t bs, int64_t* slots,
                                        int64_t slot_capacity, int32_t* lens_out,
                                        int32_t* cow_src, int32_t* cow_dst,
                                        int32_t* cow_count, int32_t* status,
                                        hipStream_t stream) {
  reserve_shared_kernel<<<1, kThreads, 0, stream>>>(stack, top, capacity, refcount, tables,
                                                    max_blocks, lens, new_tokens, batch, bs,
                                                    slots, lens_out, cow_src, cow_dst,
                                                    cow_count, status, slot_capacity);
  return hipGetLastError();
}

hipError_t launch_blocks_release_shared(int32_t* stack, int32_t* top, int64_t capacity,
                                        int32_t* refcount, const int32_t* tables,
                                        int32_t max_blocks, const int32_t* lens,
                                        const int32_t* mask, int32_t batch, int32_t bs,
                                        int32_t* lens_out, int32_t* status,
                                        hipStream_t stream) {
  release_shared_kernel<<<1, kThreads, 0, stream>>>(stack, top, capacity, refcount, tables,
                                                    max_blocks, lens, mask, batch, bs, lens_out,
                                                    status);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(uint8_t* const base[6], const int64_t per_block[6],
                              const int32_t* src, const int32_t* dst, const int32_t* count,
                              int32_t max_pairs, int64_t num_blocks, hipStream_t stream) {
  CopyPlanes cp;
  for (int i = 0; i < 6; ++i) {
    cp.base[i] = base[i];
    cp.per_block[i] = base[i] ? per_block[i] : 0;
  }
  copy_blocks_kernel<<<dim3(max_pairs, 6), 256, 0, stream>>>(cp, src, dst, count, num_blocks);
  return hipGetLastError();
}

hipError_t launch_pack_blocks(uint8_t* const base[6], const int64_t per_block[6],
                              const int32_t* ids, int32_t n, uint8_t* packed, bool pack,
                              int64_t num_blocks, hipStream_t stream) {
  PackPlanes pp;
  int64_t off = 0;
  for (int i = 0; i < 6; ++i) {
    pp.base[i] = base[i];
    pp.per_block[i] = base[i] ? per_block[i] : 0;
    pp.offset[i] = off;
    off += pp.per_block[i];
  }
  pp.pack_bytes = off;
  if (pack)
    pack_kernel<true><<<dim3(n, 6), 256, 0, stream>>>(pp, ids, packed, num_blocks);
  else
    pack_kernel<false><<<dim3(n, 6), 256, 0, stream>>>(pp, ids, packed, num_blocks);
  return hipGetLastError();
}

}  // namespace kvq
