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

namespace kvq {
namespace {

constexpr int kThreads = 1024;

// Block-wide exclusive scan of one int64 per thread; returns the prefix and
// writes the total to *total (all threads).
__device__ int64_t block_exclusive_scan(int64_t v, int64_t* total, int64_t* sh) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    int64_t add = tid >= off ? sh[tid - off] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int64_t incl = sh[tid];
  *total = sh[kThreads - 1];
  __syncthreads();
  return incl - v;
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
    int64_t* slots, int32_t* lens_out, int32_t* status, int64_t capacity) {
  __shared__ int64_t sh[kThreads];
  __shared__ int ok_sh;
  const int tid = threadIdx.x;
  // a top outside [0, capacity] (a broken precondition) is cut to it
  const int64_t top0 = min(max((int64_t)*top, (int64_t)0), capacity);
  // pass 1: total need and table capacity check
  if (tid == 0) ok_sh = 1;
  __syncthreads();
  int64_t total_need = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    int64_t need = 0;
    if (b < batch) {
      const int64_t have = ceil_div(lens[b], bs);
      const int64_t want = ceil_div((int64_t)lens[b] + new_tokens[b], bs);
      if (want > max_blocks) ok_sh = 0;
      need = want - have;
    }
    int64_t chunk_total;
    block_exclusive_scan(need, &chunk_total, sh);
    total_need += chunk_total;
  }
  __syncthreads();
  if (!ok_sh || total_need > top0) {
    if (tid == 0) *status = KVQ_ERR_OUT_OF_BLOCKS;
    return;
  }
  // pass 2: take blocks and write slots
  int64_t boff = 0, toff = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    int64_t have = 0, need = 0, n = 0, L = 0;
    if (b < batch) {
      L = lens[b];
      n = new_tokens[b];
      have = ceil_div(L, bs);
      need = ceil_div(L + n, bs) - have;
    }
    int64_t ctot, ttot;
    const int64_t bpre = block_exclusive_scan(need, &ctot, sh) + boff;
    const int64_t tpre = block_exclusive_scan(n, &ttot, sh) + toff;
    if (b < batch) {
      int32_t* row = tables + (int64_t)b * max_blocks;
      for (int64_t k = 0; k < need; ++k) row[have + k] = stack[top0 - bpre - need + k];
      for (int64_t k = 0; k < n; ++k) {
        const int64_t pos = L + k;
        slots[tpre + k] = (int64_t)row[pos / bs] * bs + pos % bs;
      }
      if (lens_out) lens_out[b] = (int32_t)(L + n);
    }
    boff += ctot;
    toff += ttot;
    __syncthreads();
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
  int64_t off = 0;
  for (int base = 0; base < batch; base += kThreads) {
    const int b = base + tid;
    const bool rel = b < batch && mask[b];
    const int64_t nb = rel ? min(ceil_div(lens[b], bs), (int64_t)max_blocks) : 0;
    int64_t t;
    const int64_t pre = block_exclusive_scan(nb, &t, sh) + off;
    for (int64_t k = 0; k < nb; ++k) stack[top0 + pre + k] = tables[(int64_t)b * max_blocks + k];
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

}  // namespace

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
                                 int32_t* lens_out, int32_t* status,
                                 hipStream_t stream) {
  reserve_kernel<<<1, kThreads, 0, stream>>>(stack, top, tables, max_blocks, lens,
                                             new_tokens, batch, bs, slots, lens_out,
                                             status, capacity);
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

}  // namespace kvq
