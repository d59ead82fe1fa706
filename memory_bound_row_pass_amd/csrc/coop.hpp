// The exchange of the one-pass split-row kernels: the workgroups of a row,
// one per segment, post their segment's partial state and wait for the
// others' (split.hip, split_norm.hip).
//
// Work items are handed out in start order: a workgroup takes the next
// ticket from a device-scope counter when it starts, and ticket w is row
// w / nseg, segment w % nseg. So the started workgroups always hold the
// lowest tickets, every row below the lowest unfinished one has finished,
// and that row's missing segments only need free room on the device for
// their workgroups (rows of at most kCoopMaxSegments segments): the waits
// end however the hardware orders, places or delays the workgroups.
// Posting: a state is one or two 64-bit words, each written with one
// device-scope atomic store into the segment's slot of the row; the slots
// are zeroed before the launch and the kernels choose words that are never
// zero once posted. Such stores go through to the level all XCDs share
// without the whole-L2 write-back of a device-scope release fence, and a
// reader sees a word either unposted or whole. Waiting: lane NWD j + f of
// wave 0 reads word f of segment j (64 / NWD segments per round) with
// device-scope atomic loads until every word is posted. Bounded: after
// spin_limit polls (each after a short sleep), or once another wait has
// given up (the abort word), a workgroup takes NaN for the missing words —
// its outputs of that row are NaN — and sets the abort word; the kernel
// always ends.
// Workspace (coop_workspace_bytes): ctl[0] the ticket counter, ctl[1] the
// abort word (16 bytes), then the slots [rows][nseg][2] words.
#pragma once

#include "fr_device.hpp"
#include "fr_kernels.hpp"

namespace fr {

__device__ __forceinline__ uint64_t coop_word(float lo, float hi) {
  return ((uint64_t)__builtin_bit_cast(uint32_t, hi) << 32) | __builtin_bit_cast(uint32_t, lo);
}

// This workgroup's work item (uniform). One barrier; `slot` is LDS.
__device__ __forceinline__ int64_t coop_ticket(uint32_t* ctl, uint32_t* slot) {
  if (threadIdx.x == 0) *slot = __hip_atomic_fetch_add(ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  lds_barrier();
  return __builtin_amdgcn_readfirstlane(*slot);
}

// Threads 0 .. NWD-1 post word f of segment sg into the row's slots.
template <int NWD>
__device__ __forceinline__ void coop_post(uint64_t* row_slots, int sg, uint64_t w0, uint64_t w1) {
  if (threadIdx.x < NWD)
    __hip_atomic_store(row_slots + (size_t)sg * 2 + threadIdx.x, threadIdx.x == 0 ? w0 : w1,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wave 0: waits for word f < NWD of segment j < nseg of the row's slots and
// leaves its halves in team[j][2 f] (low) and team[j][2 f + 1] (high), NaN
// for a word that did not arrive. The caller's barrier publishes team.
// Returns (uniformly) whether every word arrived.
template <int NWD>
__device__ __forceinline__ bool coop_wait(const uint64_t* row_slots, int nseg, uint32_t* abort_word,
                                          int spin_limit, int lane, float (*team)[4]) {
  constexpr int PER = 64 / NWD;  // segments per round
  const int f = lane % NWD;
  bool all = true;
  for (int j0 = 0; j0 < nseg; j0 += PER) {
    const int j = j0 + lane / NWD;
    const bool live = j < nseg;
    uint64_t word = 0;
    bool have = !live;
    for (int spins = 0;; ++spins) {
      if (!have) {
        word = __hip_atomic_load(row_slots + (size_t)j * 2 + f, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        have = word != 0;
      }
      if (__builtin_amdgcn_ballot_w64(!have) == 0) break;
      bool give_up = spins >= spin_limit;
      if ((spins & 15) == 15)
        give_up = give_up ||
                  __hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0;
      if (__builtin_amdgcn_readfirstlane((int)give_up)) {
        if (lane == 0) __hip_atomic_store(abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        all = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (live) {
      team[j][2 * f] = have ? __builtin_bit_cast(float, (uint32_t)word) : __builtin_nanf("");
      team[j][2 * f + 1] = have ? __builtin_bit_cast(float, (uint32_t)(word >> 32)) : __builtin_nanf("");
    }
  }
  return all;
}

// Zeroes the one-pass workspace of rows x nseg work items (split.hip).
hipError_t launch_coop_clear(void* ws, int64_t rows, int nseg, hipStream_t s);

}  // namespace fr
