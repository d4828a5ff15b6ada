// Internal declarations shared by the host-side sources of libmoe.
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

#include "moe.h"

namespace moe {

// Thread-local last-error string behind moe_last_error().
void set_error(const std::string& msg);
void clear_error();
moe_status fail(moe_status st, const std::string& msg);

// Config validation shared by every entry point. Returns an empty string when
// valid, else the reason.
std::string check_config(const moe_config* cfg);

// Chunk geometry of a code row: a chunk is 16 bytes of codes
// (32 int4 or 16 int8 elements).
inline int chunks_per_row(int k_elems, int bits) { return k_elems * bits / 128; }

size_t record_bytes(const moe_config& c, int inter);
size_t record_stride(const moe_config& c, int inter);

struct RecordLayout {
  size_t gate_codes, up_codes, down_codes, gate_sc, up_sc, down_sc, end;
};
RecordLayout record_layout(const moe_config& c, int inter);

// IEEE binary32 -> binary16, round to nearest, ties to even (bit pattern).
uint16_t f32_to_f16_rne(float f);
float f16_to_f32(uint16_t h);

}  // namespace moe
