// QUOKA_DEBUG mode and quoka_check_selection: device-side checks of the
// entry points' preconditions and of the selection's result (debug.hip).
#pragma once

#include <stdint.h>

#include "internal.h"

namespace quoka {

// one result slot per checked argument
enum DebugSlot {
  kDbgQ = 0, kDbgKHist, kDbgVHist, kDbgKChunk, kDbgVChunk, kDbgKSel, kDbgVSel,
  kDbgSelIn, kDbgSelOut, kDbgK, kDbgV, kDebugSlots
};

// what a DebugItem checks
enum DebugKind {
  kDebugRowsAll = 0,   // every element finite
  kDebugRowsSel,       // [S, Hkv, kv_budget, d]: rows b < B_eff finite
  kDebugIdxInput,      // [S, Hkv, kv_budget] int32: -1 or in [0, L_s)
  kDebugIdxSelection,  // [S, Hkv, kv_budget] int32: the selection's layout
};

struct DebugItem {
  const void* ptr;
  int64_t count;  // elements
  int kind;       // DebugKind
  int slot;       // DebugSlot
};

// QUOKA_DEBUG is set (and not "0"); read on every call.
bool debug_mode();

// The device offset arrays hold the host copies' values (QUOKA_EINVAL if not).
quoka_status debug_offsets(const Problem& p);

// Runs the checks on stream st and waits for them. The first failure, in
// item order, gives QUOKA_EINVAL (an argument) or QUOKA_ECHECK (a result).
// Calls are serialised: every call on a device shares one result array.
quoka_status debug_run(const Problem& p, const DebugItem* items, int n, hipStream_t st);

}  // namespace quoka
