// Process-wide tuning settings: which scan order a call takes, the chunk
// length of the chunked order, and chains per lane.  They start from the
// environment (MSSM_SCAN_DESIGN, MSSM_CHUNK_LEN, MSSM_CPL), read once, the
// first time any setting is needed; mssm_set_tuning changes them afterwards.
// Calls never read the environment themselves: getenv costs host time on
// every launch and races with a thread that changes the environment.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include "mssm_internal.h"

namespace mssm {

namespace {

struct Settings {
  std::atomic<int64_t> value[3];
  Settings() {
    int64_t order = MSSM_ORDER_AUTO;
    if (const char* e = std::getenv("MSSM_SCAN_DESIGN")) {
      if (std::strcmp(e, "chunked") == 0) order = MSSM_ORDER_CHUNKED;
      if (std::strcmp(e, "chain") == 0) order = MSSM_ORDER_SINGLE_PASS;
    }
    int64_t chunk = 0;
    if (const char* e = std::getenv("MSSM_CHUNK_LEN")) {
      const long long v = std::atoll(e);
      if (v > 0) chunk = v;
    }
    int64_t cpl = 0;
    if (const char* e = std::getenv("MSSM_CPL")) {
      const int v = std::atoi(e);
      if (v == 1 || v == 2) cpl = v;
    }
    value[MSSM_TUNE_SCAN_ORDER].store(order);
    value[MSSM_TUNE_CHUNK_LEN].store(chunk);
    value[MSSM_TUNE_CHAINS_PER_LANE].store(cpl);
  }
};

// built on first use (C++ guarantees one thread-safe initialisation)
Settings& settings() {
  static Settings s;
  return s;
}

}  // namespace

int64_t tuning(mssm_tuning key) { return settings().value[key].load(std::memory_order_relaxed); }

}  // namespace mssm

extern "C" {

mssm_status mssm_set_tuning(mssm_tuning key, int64_t value) {
  switch (key) {
    case MSSM_TUNE_SCAN_ORDER:
      if (value != MSSM_ORDER_AUTO && value != MSSM_ORDER_CHUNKED &&
          value != MSSM_ORDER_SINGLE_PASS)
        return MSSM_ERROR_INVALID_VALUE;
      break;
    case MSSM_TUNE_CHUNK_LEN:
      if (value < 0) return MSSM_ERROR_INVALID_VALUE;
      break;
    case MSSM_TUNE_CHAINS_PER_LANE:
      if (value < 0 || value > 2) return MSSM_ERROR_INVALID_VALUE;
      break;
    default:
      return MSSM_ERROR_INVALID_VALUE;
  }
  mssm::settings().value[key].store(value, std::memory_order_relaxed);
  return MSSM_SUCCESS;
}

mssm_status mssm_get_tuning(mssm_tuning key, int64_t* value) {
  if (!value) return MSSM_ERROR_INVALID_VALUE;
  if (key != MSSM_TUNE_SCAN_ORDER && key != MSSM_TUNE_CHUNK_LEN &&
      key != MSSM_TUNE_CHAINS_PER_LANE)
    return MSSM_ERROR_INVALID_VALUE;
  *value = mssm::tuning(key);
  return MSSM_SUCCESS;
}

}  // extern "C"
