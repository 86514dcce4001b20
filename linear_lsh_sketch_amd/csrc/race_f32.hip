// float32 instantiations of the RACE Attention launch sequences.
#include "race_dispatch.hpp"

namespace race {
template race_status_t dispatch<true>(const Shape&, const Derived&, const WsLayout&, const Call&);
}
