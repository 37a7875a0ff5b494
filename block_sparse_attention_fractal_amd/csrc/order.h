// Host-side token order tables (plain C++, no HIP calls).
#pragma once
#include <stdint.h>
#include <string>

#include "bsa.h"
#include "geom.h"

namespace bsa {

// table[f] = original (t, h, w) row-major index of the token at position f
// (L entries, host memory).  Returns a bsa status and a message on failure.
int order_table(const Geom& g, int order, int32_t* table, std::string* msg);

}  // namespace bsa
