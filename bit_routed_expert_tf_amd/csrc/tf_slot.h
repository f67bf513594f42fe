// Slot-cache internals used by the layer entry point.
#pragma once
#include "tf_internal.h"

tf_status tf_slot_check_layer(const tf_slot_cache *c, const tf_moe_layer *L, int32_t layer);
hipEvent_t tf_slot_fill_event(tf_slot_cache *c);
const int32_t *tf_slot_map(const tf_slot_cache *c, int32_t layer);
const uint8_t *tf_slot_pool(const tf_slot_cache *c, int32_t layer);
