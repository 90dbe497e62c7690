// Checks of the device-side inputs the attention and cache calls take on trust.
//
// The paged calls never read their index arrays back to the host (that would need
// a synchronisation), so a block id outside the pool, a length past the table, a
// repeated write slot or overlapping copy pairs are undefined behaviour there.
// These kernels read the same arrays and only compare values -- no id is ever
// used as an address -- and OR a bit per kind of violation into a caller-owned
// device word (PA_CHECK_* in pa.h).  They are a debugging aid: the slot and pair
// checks compare every pair of entries (quadratic in the count).
//
// What is checked follows the addressing the pages describe (5688vip chapter 3,
// section 3.2: logical block p / block_size of a request is found through its
// block table; uml.org.cn "Prefix Sharing": a copied page is a fresh page, so a
// copy never writes a page another copy of the same step reads).
#include "pa_device.h"
#include "pa_launch.h"

namespace pa {

// One workgroup per sequence.
__global__ __launch_bounds__(64) void pa_check_tables_kernel(CheckTablesArgs a) {
  const int s = blockIdx.x;
  const int n = a.lens[s];
  int f = 0;
  if (threadIdx.x == 0) {
    if (n < 1 || n > a.max_len || (int64_t)n > (int64_t)a.mbps * a.block_size) f |= PA_CHECK_LEN;
    if (a.qsl != nullptr) {
      const int q0 = a.qsl[s], q1 = a.qsl[s + 1];
      if ((s == 0 && q0 != 0) || q1 - q0 < 1 || q1 - q0 > n) f |= PA_CHECK_QSL;
    }
  }
  // the used part of the table row: entries 0 .. ceil(n / block_size) - 1
  const int64_t used = n > 0 ? ((int64_t)n + a.block_size - 1) / a.block_size : 0;
  const int nb = (int)(used < a.mbps ? used : a.mbps);
  const int32_t *row = a.bt + (int64_t)s * a.mbps;
  for (int j = threadIdx.x; j < nb; j += blockDim.x) {
    const int32_t b = row[j];
    if (b < 0 || (int64_t)b >= a.num_blocks) f |= PA_CHECK_BLOCK;
  }
  if (f) atomicOr(a.flags, f);
}

// Thread i: its slot's range, and equality with every later slot.
__global__ __launch_bounds__(256) void pa_check_slots_kernel(const int64_t *slots, int32_t n,
                                                             int64_t num_slots, int32_t *flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t x = slots[i];
  int f = 0;
  if (x >= num_slots) f |= PA_CHECK_SLOT;
  if (x >= 0)
    for (int j = i + 1; j < n; ++j)
      if (slots[j] == x) {
        f |= PA_CHECK_SLOT_DUP;
        break;
      }
  if (f) atomicOr(flags, f);
}

// Thread i: pair i's ids in range, its destination unique, its source no pair's
// destination.
__global__ __launch_bounds__(256) void pa_check_pairs_kernel(const int32_t *pairs, int32_t n,
                                                             int64_t num_blocks, int32_t *flags) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
  int f = 0;
  if (src < 0 || (int64_t)src >= num_blocks || dst < 0 || (int64_t)dst >= num_blocks)
    f |= PA_CHECK_PAIR;
  for (int j = 0; j < n; ++j) {
    const int32_t dj = pairs[2 * j + 1];
    if ((j > i && dj == dst) || dj == src) {
      f |= PA_CHECK_PAIR;
      break;
    }
  }
  if (f) atomicOr(flags, f);
}

hipError_t launch_check_tables(const CheckTablesArgs &a, int32_t num_seqs, hipStream_t st) {
  hipLaunchKernelGGL(pa_check_tables_kernel, dim3(num_seqs), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_check_slots(const int64_t *slots, int32_t n, int64_t num_slots, int32_t *flags,
                              hipStream_t st) {
  hipLaunchKernelGGL(pa_check_slots_kernel, dim3((n + 255) / 256), dim3(256), 0, st, slots, n,
                     num_slots, flags);
  return hipGetLastError();
}

hipError_t launch_check_pairs(const int32_t *pairs, int32_t n, int64_t num_blocks,
                              int32_t *flags, hipStream_t st) {
  hipLaunchKernelGGL(pa_check_pairs_kernel, dim3((n + 255) / 256), dim3(256), 0, st, pairs, n,
                     num_blocks, flags);
  return hipGetLastError();
}

}  // namespace pa
